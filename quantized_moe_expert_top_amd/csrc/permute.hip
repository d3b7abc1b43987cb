// Grouping of the T*k routed slots by expert: a stable counting sort.
//
// histogram of expert ids -> exclusive prefix sum -> stable scatter into
// expert-contiguous order ("Performance and verification", section "Why it is
// fast": a batch reads every routed expert it calls once, which needs the
// batch's rows grouped per expert). Integer work only, so every output is
// exact and deterministic (integer LDS atomics for the counts, nothing else).
//
// Stability inside a round of 64 slots comes from a wave-level "match": lanes
// holding the same expert id are found with one ballot per id bit; a lane's
// rank is the number of matching lanes below it, and per-wave counts kept in
// LDS order the waves of the block. Up to 8192 slots (E <= 512) one block of
// 1024 threads does everything in one launch; beyond that,
// chunks of 1024 slots are handled by one block each, and a block's base per
// expert is the count of that expert in all earlier chunks (a column prefix
// sum over the per-chunk histograms).
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

// Block-wide exclusive scan of one value per thread (NTHR threads).
template <int NTHR>
__device__ __forceinline__ int block_excl_scan_n(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == kWave - 1) wave_tot[w] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < NTHR / kWave; ++i) {
    const int t = wave_tot[i];
    if (i < w) before += t;
    total += t;
  }
  __syncthreads();
  return before + incl - v;
}

// counts[e] (LDS) -> offsets (global, [E+1]) and run[e] (LDS, = offsets[e]);
// the active list and its length.
template <int NTHR>
__device__ void offsets_and_active(const int* counts, int* run, int E, int R, int* wave_tot,
                                   int* offsets, int* active, int* n_active) {
  if (E <= 4 * kWave && R < (1 << 16)) {   // uniform
    // wave 0 alone, four experts a lane, with no block barrier: one scan of
    // count (low 16 bits, sum <= R) and active flag (high bits) packed together
    if (threadIdx.x < kWave) {
      const int lane = threadIdx.x;
      int c[4], v = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = lane * 4 + i;
        c[i] = e < E ? counts[e] : 0;
        v += c[i] + (c[i] > 0 ? (1 << 16) : 0);
      }
      const int incl = wave_incl_scan(v);
      const int excl = incl - v;
      int oc = excl & 0xFFFF, of = excl >> 16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = lane * 4 + i;
        if (e < E) {
          run[e] = oc;
          offsets[e] = oc;
          if (c[i]) active[of] = e;
        }
        oc += c[i];
        of += c[i] > 0;
      }
      if (lane == kWave - 1) {
        offsets[E] = R;
        *n_active = incl >> 16;
      }
    }
    return;
  }
  const int ept = (E + NTHR - 1) / NTHR;  // <= 4
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
  int oc = block_excl_scan_n<NTHR>(sc, wave_tot, tot_c);
  int of = block_excl_scan_n<NTHR>(sf, wave_tot, tot_f);
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

// The ids of slots base + r * NTHR + tid, r < MAXR, as sort keys (E past the
// end of [base, R)), loaded together (clamped addresses, no branches) so
// their latencies overlap. With no slot at or after base (an empty batch,
// where ids may be NULL) nothing is read.
template <int NTHR, int MAXR>
__device__ __forceinline__ void load_keys(const int* __restrict__ ids, int R, int E, int base,
                                          uint32_t (&keys)[MAXR]) {
  if (base >= R) {   // uniform across the block
#pragma unroll
    for (int r = 0; r < MAXR; ++r) keys[r] = static_cast<uint32_t>(E);
    return;
  }
  int raw[MAXR];
#pragma unroll
  for (int r = 0; r < MAXR; ++r) raw[r] = ids[min(base + r * NTHR + static_cast<int>(threadIdx.x), R - 1)];
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    const int f = base + r * NTHR + threadIdx.x;
    keys[r] = f < R ? static_cast<uint32_t>(clamp_id(raw[r], E)) : static_cast<uint32_t>(E);
  }
}

// Stable scatter of slots base + r * NTHR + tid (r < MAXR, slot < R) in
// rounds of NTHR, given their keys and run[e] = first free grouped position
// of expert e. wc[NTHR / 64 * E] must be zero on entry and is left zero.
template <int NTHR, int MAXR>
__device__ void scatter_keys(const uint32_t (&keys)[MAXR], int R, int E, int nbits, int base,
                             int* run, int* wc, int* __restrict__ sorted_slot,
                             int* __restrict__ slot_pos) {
  constexpr int NW = NTHR / kWave;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid >> 6;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    if (base + r * NTHR >= R) break;   // uniform across the block
    const int f = base + r * NTHR + tid;
    const bool valid = f < R;
    const uint32_t key = keys[r];
    const uint64_t m = wave_match(key, nbits);
    const int rank = __popcll(m & below);
    const bool leader = rank == 0;
    if (valid && leader) wc[w * E + key] = __popcll(m);
    __syncthreads();
    int pre = 0, tot = 0;
    if (valid) {
#pragma unroll
      for (int v = 0; v < NW; ++v) {
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

// Everything in one block of NTHR threads (R <= kChunk with 256 threads, up
// to kSingleMaxR with 1024): one launch instead of three. Wave w owns the
// contiguous slots [w * SPW, (w + 1) * SPW) and walks them in rounds of 64 in
// increasing order, so a slot's stable position is its expert's offset + the
// expert's slots in earlier waves + those earlier in its own wave. Each wave
// keeps its own per-expert counts in LDS (no atomics, no barrier between
// rounds: a wave's LDS operations complete in order); one pass over the
// counts turns them into per-wave prefixes.
template <int NTHR, int MAXR>
__global__ __launch_bounds__(NTHR) void permute_small_kernel(
    const int* __restrict__ ids, int R, int E, int* __restrict__ offsets,
    int* __restrict__ sorted_slot, int* __restrict__ slot_pos, int* __restrict__ active,
    int* __restrict__ n_active) {
  constexpr int NW = NTHR / kWave;
  extern __shared__ __attribute__((aligned(16))) int sm[];
  int* counts = sm;            // [E]
  int* run = counts + E;       // [E]
  int* wc = run + E;           // [NW][E]: per-wave counts, then prefixes over waves
  __shared__ int wave_tot[NW];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid >> 6;
  const int SPW = kWave * ((R + kWave * NW - 1) / (kWave * NW));  // <= 64 * MAXR
  const int f0 = w * SPW;
  // every slot's id is read from memory once, all loads in flight together
  int raw[MAXR];
  if (R > 0) {   // uniform; with no slot, ids may be NULL
#pragma unroll
    for (int r = 0; r < MAXR; ++r) raw[r] = ids[min(f0 + r * kWave + lane, R - 1)];
  }
  uint32_t keys[MAXR];
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    const int f = f0 + r * kWave + lane;
    keys[r] = (R > 0 && r * kWave < SPW && f < R) ? static_cast<uint32_t>(clamp_id(raw[r], E))
                                                  : static_cast<uint32_t>(E);
  }
  for (int i = tid; i < NW * E; i += NTHR) wc[i] = 0;
  __syncthreads();
  const int nbits = id_bits(E);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  int lp[MAXR];   // position among this wave's slots of the same expert
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    lp[r] = 0;
    if (r * kWave >= SPW) continue;   // uniform
    const uint32_t key = keys[r];
    const uint64_t m = wave_match(key, nbits);
    const int rank = __popcll(m & below);
    const bool real = key < static_cast<uint32_t>(E);
    const int before = real ? wc[w * E + key] : 0;
    lp[r] = before + rank;
    if (real && rank == 0) wc[w * E + key] = before + __popcll(m);
  }
  __syncthreads();
  for (int e = tid; e < E; e += NTHR) {
    int acc = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const int c = wc[v * E + e];
      wc[v * E + e] = acc;
      acc += c;
    }
    counts[e] = acc;
  }
  __syncthreads();
  offsets_and_active<NTHR>(counts, run, E, R, wave_tot, offsets, active, n_active);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    const int f = f0 + r * kWave + lane;
    if (r * kWave < SPW && f < R) {
      const uint32_t key = keys[r];
      const int pos = run[key] + wc[w * E + key] + lp[r];
      sorted_slot[pos] = f;
      slot_pos[f] = pos;
    }
  }
}

__global__ __launch_bounds__(kThreads) void permute_hist_kernel(const int* __restrict__ ids,
                                                                int R, int E,
                                                                int* __restrict__ hist) {
  extern __shared__ __attribute__((aligned(16))) int counts[];
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
  extern __shared__ __attribute__((aligned(16))) int sm[];
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
  offsets_and_active<kThreads>(counts, run, E, R, wave_tot, offsets, active, n_active);
}

__global__ __launch_bounds__(kThreads) void permute_scatter_kernel(
    const int* __restrict__ ids, const int* __restrict__ bases,
    const int* __restrict__ offsets, int R, int E, int* __restrict__ sorted_slot,
    int* __restrict__ slot_pos) {
  extern __shared__ __attribute__((aligned(16))) int sm[];
  int* run = sm;          // [E]
  int* wc = sm + E;       // [kWaves * E]
  for (int e = threadIdx.x; e < E; e += kThreads)
    run[e] = offsets[e] + bases[static_cast<size_t>(blockIdx.x) * E + e];
  for (int i = threadIdx.x; i < kWaves * E; i += kThreads) wc[i] = 0;
  __syncthreads();
  uint32_t keys[kChunk / kThreads];
  load_keys<kThreads, kChunk / kThreads>(ids, R, E, blockIdx.x * kChunk, keys);
  scatter_keys<kThreads, kChunk / kThreads>(keys, R, E, id_bits(E), blockIdx.x * kChunk, run, wc,
                                            sorted_slot, slot_pos);
}

}  // namespace

// the one-block path at 1024 threads: R <= kSingleMaxR and E <= kSingleMaxE
// (its LDS, (2 + 16) * E ints, stays within 64 KiB)
constexpr int kSingleMaxR = 8192;
constexpr int kSingleMaxE = 512;
static bool single_block(long long R, int E) {
  return R <= kChunk || (R <= kSingleMaxR && E <= kSingleMaxE);
}

size_t permute_workspace_bytes(int T, int E, int k) {
  const long long R = static_cast<long long>(T) * k;
  if (single_block(R, E)) return 0;
  const long long NB = (R + kChunk - 1) / kChunk;
  return static_cast<size_t>(2 * NB * E) * sizeof(int);
}

hipError_t launch_permute(const int* ids, int T, int E, int k, int* offsets, int* sorted_slot,
                          int* slot_pos, int* active, int* n_active, void* ws, hipStream_t s) {
  const int R = T * k;
  if (R <= kChunk) {
    const size_t lds = static_cast<size_t>(2 + kWaves) * E * sizeof(int);
    permute_small_kernel<kThreads, kChunk / kThreads><<<1, kThreads, lds, s>>>(
        ids, R, E, offsets, sorted_slot, slot_pos, active, n_active);
    return hipGetLastError();
  }
  if (single_block(R, E)) {
    const size_t lds = static_cast<size_t>(2 + 1024 / kWave) * E * sizeof(int);
    permute_small_kernel<1024, kSingleMaxR / 1024><<<1, 1024, lds, s>>>(
        ids, R, E, offsets, sorted_slot, slot_pos, active, n_active);
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
