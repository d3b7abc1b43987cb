// Grouping of the T*k routed slots by expert: a stable counting sort.
//
// histogram of expert ids -> exclusive prefix sum -> stable scatter into
// expert-contiguous order ("Performance and verification", section "Why it is
// fast": a batch reads every routed expert it calls once, which needs the
// batch's rows grouped per expert). Integer work only, so every output is
// exact and deterministic (integer LDS atomics for the counts, nothing else).
//
// Stability inside a 256-slot round comes from a wave-level "match": lanes
// holding the same expert id are found with one ballot per id bit; a lane's
// rank is the number of matching lanes below it, and per-wave counts kept in
// LDS order the four waves of the block. Chunks of 1024 slots are handled by
// one block each; a block's base per expert is the count of that expert in
// all earlier chunks (a column prefix sum over the per-chunk histograms).
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 1024;  // slots per block
constexpr int kWaves = kThreads / kWave;

// Ids outside [0, E) are outside the contract; clamping keeps every access
// inside its buffer.
__device__ __forceinline__ int clamp_id(int id, int E) {
  return static_cast<unsigned>(id) < static_cast<unsigned>(E) ? id : E - 1;
}

__device__ __forceinline__ uint64_t wave_match(uint32_t key, int nbits) {
  uint64_t m = ~0ull;
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1u;
    const uint64_t v = __ballot(bit);
    m &= bit ? v : ~v;
  }
  return m;
}

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  return v;
}

// Block-wide exclusive scan of one value per thread (256 threads).
__device__ __forceinline__ int block_excl_scan(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == kWave - 1) wave_tot[w] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const int t = wave_tot[i];
    if (i < w) before += t;
    total += t;
  }
  __syncthreads();
  return before + incl - v;
}

// counts[e] (LDS) -> offsets (global, [E+1]) and run[e] (LDS, = offsets[e]);
// the active list and its length.
__device__ void offsets_and_active(const int* counts, int* run, int E, int R, int* wave_tot,
                                   int* offsets, int* active, int* n_active) {
  const int ept = (E + kThreads - 1) / kThreads;  // <= 4
  const int e0 = threadIdx.x * ept;
  int c[4], f[4], sc = 0, sf = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = e0 + i;
    c[i] = (i < ept && e < E) ? counts[e] : 0;
    f[i] = c[i] > 0 ? 1 : 0;
    sc += c[i];
    sf += f[i];
  }
  int tot_c, tot_f;
  int oc = block_excl_scan(sc, wave_tot, tot_c);
  int of = block_excl_scan(sf, wave_tot, tot_f);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = e0 + i;
    if (i < ept && e < E) {
      run[e] = oc;
      offsets[e] = oc;
      if (f[i]) active[of] = e;
    }
    oc += c[i];
    of += f[i];
  }
  if (threadIdx.x == 0) {
    offsets[E] = R;
    *n_active = tot_f;
  }
}

// Stable scatter of slots [base, base + kChunk) given run[e] = first free
// grouped position of expert e. wc[kWaves * E] must be zero on entry and is
// left zero.
__device__ void scatter_chunk(const int* __restrict__ ids, int R, int E, int nbits, int base,
                              int* run, int* wc, int* __restrict__ sorted_slot,
                              int* __restrict__ slot_pos) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid >> 6;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int r = 0; r < kChunk / kThreads; ++r) {
    const int f = base + r * kThreads + tid;
    const bool valid = f < R;
    const uint32_t key = valid ? static_cast<uint32_t>(clamp_id(ids[f], E)) : static_cast<uint32_t>(E);
    const uint64_t m = wave_match(key, nbits);
    const int rank = __popcll(m & below);
    const bool leader = rank == 0;
    if (valid && leader) wc[w * E + key] = __popcll(m);
    __syncthreads();
    int pre = 0, tot = 0;
    if (valid) {
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        const int c = wc[v * E + key];
        if (v < w) pre += c;
        tot += c;
      }
      const int pos = run[key] + pre + rank;
      sorted_slot[pos] = f;
      slot_pos[f] = pos;
    }
    __syncthreads();
    if (valid && leader) {
      if (pre == 0) run[key] += tot;  // first wave holding this expert
      wc[w * E + key] = 0;
    }
    __syncthreads();
  }
}

__device__ __forceinline__ int id_bits(int E) { return 32 - __clz(E); }  // covers 0..E

// R <= kChunk: everything in one block.
__global__ __launch_bounds__(kThreads) void permute_small_kernel(
    const int* __restrict__ ids, int R, int E, int* __restrict__ offsets,
    int* __restrict__ sorted_slot, int* __restrict__ slot_pos, int* __restrict__ active,
    int* __restrict__ n_active) {
  extern __shared__ int sm[];
  int* counts = sm;            // [E]
  int* run = counts + E;       // [E]
  int* wc = run + E;           // [kWaves * E]
  __shared__ int wave_tot[kWaves];
  for (int i = threadIdx.x; i < (2 + kWaves) * E; i += kThreads) sm[i] = 0;
  __syncthreads();
  for (int f = threadIdx.x; f < R; f += kThreads) atomicAdd(&counts[clamp_id(ids[f], E)], 1);
  __syncthreads();
  offsets_and_active(counts, run, E, R, wave_tot, offsets, active, n_active);
  __syncthreads();
  scatter_chunk(ids, R, E, id_bits(E), 0, run, wc, sorted_slot, slot_pos);
}

__global__ __launch_bounds__(kThreads) void permute_hist_kernel(const int* __restrict__ ids,
                                                                int R, int E,
                                                                int* __restrict__ hist) {
  extern __shared__ int counts[];
  for (int i = threadIdx.x; i < E; i += kThreads) counts[i] = 0;
  __syncthreads();
  const int base = blockIdx.x * kChunk;
  for (int i = threadIdx.x; i < kChunk; i += kThreads) {
    const int f = base + i;
    if (f < R) atomicAdd(&counts[clamp_id(ids[f], E)], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads)
    hist[static_cast<size_t>(blockIdx.x) * E + e] = counts[e];
}

// One block: column prefix sums over chunks, expert offsets, active list.
// bases[b][e] = rows of expert e in chunks before b (within-expert prefix);
// the scatter adds the expert's offset. Loads go out eight at a time.
__global__ __launch_bounds__(kThreads) void permute_scan_kernel(
    const int* __restrict__ hist, int* __restrict__ bases, int NB, int R, int E,
    int* __restrict__ offsets, int* __restrict__ active, int* __restrict__ n_active) {
  extern __shared__ int sm[];
  int* counts = sm;       // [E]
  int* run = sm + E;      // [E]
  __shared__ int wave_tot[kWaves];
  for (int e = threadIdx.x; e < E; e += kThreads) {
    int acc = 0, b = 0;
    for (; b + 8 <= NB; b += 8) {
      int hv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) hv[u] = hist[static_cast<size_t>(b + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        bases[static_cast<size_t>(b + u) * E + e] = acc;
        acc += hv[u];
      }
    }
    for (; b < NB; ++b) {
      const size_t i = static_cast<size_t>(b) * E + e;
      const int h = hist[i];
      bases[i] = acc;
      acc += h;
    }
    counts[e] = acc;
  }
  __syncthreads();
  offsets_and_active(counts, run, E, R, wave_tot, offsets, active, n_active);
}

__global__ __launch_bounds__(kThreads) void permute_scatter_kernel(
    const int* __restrict__ ids, const int* __restrict__ bases,
    const int* __restrict__ offsets, int R, int E, int* __restrict__ sorted_slot,
    int* __restrict__ slot_pos) {
  extern __shared__ int sm[];
  int* run = sm;          // [E]
  int* wc = sm + E;       // [kWaves * E]
  for (int e = threadIdx.x; e < E; e += kThreads)
    run[e] = offsets[e] + bases[static_cast<size_t>(blockIdx.x) * E + e];
  for (int i = threadIdx.x; i < kWaves * E; i += kThreads) wc[i] = 0;
  __syncthreads();
  scatter_chunk(ids, R, E, id_bits(E), blockIdx.x * kChunk, run, wc, sorted_slot, slot_pos);
}

}  // namespace

size_t permute_workspace_bytes(int T, int E, int k) {
  const long long R = static_cast<long long>(T) * k;
  if (R <= kChunk) return 0;
  const long long NB = (R + kChunk - 1) / kChunk;
  return static_cast<size_t>(2 * NB * E) * sizeof(int);
}

hipError_t launch_permute(const int* ids, int T, int E, int k, int* offsets, int* sorted_slot,
                          int* slot_pos, int* active, int* n_active, void* ws, hipStream_t s) {
  const int R = T * k;
  if (R <= kChunk) {
    const size_t lds = static_cast<size_t>(2 + kWaves) * E * sizeof(int);
    permute_small_kernel<<<1, kThreads, lds, s>>>(ids, R, E, offsets, sorted_slot, slot_pos,
                                                  active, n_active);
    return hipGetLastError();
  }
  const int NB = (R + kChunk - 1) / kChunk;
  int* hist = static_cast<int*>(ws);
  int* bases = hist + static_cast<size_t>(NB) * E;
  permute_hist_kernel<<<NB, kThreads, E * sizeof(int), s>>>(ids, R, E, hist);
  permute_scan_kernel<<<1, kThreads, 2 * E * sizeof(int), s>>>(hist, bases, NB, R, E, offsets,
                                                               active, n_active);
  permute_scatter_kernel<<<NB, kThreads, (1 + kWaves) * E * sizeof(int), s>>>(
      ids, bases, offsets, R, E, sorted_slot, slot_pos);
  return hipGetLastError();
}

}  // namespace moe
