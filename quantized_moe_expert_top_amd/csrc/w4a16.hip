// Grouped SwiGLU expert FFN over W4A16 g128 weights.
//
// Weight format ("Measured results", header: W4A16 g128): 4-bit codes packed
// two per byte along K (low nibble = even k), zero point 8, one fp16 scale per
// (output row, 128-wide K group); W[n,k] = (q - 8) * s[n, k/128]. Weights are
// used as stored ("Performance and verification", section "Why it is fast"):
// codes are streamed once per call and widened in registers, never expanded
// in memory (one layout serves decode and prefill: "Measured results",
// section "Memory").
//
// Dequantization trick used by both kernels: a code q placed in the low
// mantissa bits of bf16 0x4300 is exactly 128 + q, so widening a code costs
// one mask-and-or per pair. Within one 128-wide group the scale is common, so
//   sum_k x_k (q_k - 8) = sum_k x_k (128 + q_k) - sum_k x_k * 136,
// and the scale multiplies the float32 difference once per group: weights
// are never rounded. The bias term is computed by the very same instruction
// chain with every code replaced by 8 (dot2 chain at staging for the GEMV, an
// MFMA with constant B = 136 for the GEMM), so all-8 codes (a zero weight)
// give exactly zero, and rounding in the two chains is correlated.
//
// Two kernels, chosen by batch size (a fixed rule, same tolerance for both):
//  * decode (T <= 4): grouped GEMV. A block owns one routed expert and a strip
//    of output rows; LK lanes split K with coalesced 16-byte code loads, the
//    token rows live in LDS, and v_dot2_f32_bf16 does the products.
//  * prefill: grouped GEMM on bf16 MFMA (v_mfma_f32_32x32x16_bf16). A block
//    owns (expert, 32- or 64-row tile, column tile); codes go from HBM to
//    registers and are widened right into the MFMA B operand; the gathered
//    activation rows go through LDS.
// Gate/up blocks pair gate row n with up row I + n in the same lane and apply
// SwiGLU in the epilogue (h is stored bf16); down blocks write y (float32).
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "tiles.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kGemvMaxT = 4;

// 16-byte load of weight codes that are streamed once per call: the
// non-temporal hint keeps them from displacing other lines in the caches. With
// plain loads a decode_large step after a 1 GiB write took 123 us, with this
// hint 79.5 us (68 us when the memory-side cache holds no other dirty data).
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------- GEMV ----
// KIND 0: gate/up (A = x rows of the tokens, out = h bf16 [R, I]).
// KIND 1: down    (A = h rows of the expert's block, out = y float32 [R, N]).
// A block owns one routed expert and UB units of output (a unit is a gate row
// with its up row, or two down rows). Inside a wave, LK lanes split K: lane
// lk reads the 16-byte code chunks lk, lk+LK, ... of each of its two rows
// (coalesced LK*16-byte runs), so per chunk the 64 bytes of activations it
// needs are read from LDS once for both rows.
//
// Latency order: the expert id is the only thing the weight stream depends
// on, so the first batch of code chunks is requested right after it. For the
// gate/up kernel every token row of x is staged (decode has T <= 4), which
// needs no routing information; which rows belong to the expert is looked up
// while the weights are in flight. Loads are unconditional (indices clamped)
// so they issue back to back; only the arithmetic is predicated.
//
// NB: code chunks per lane per batch (= chunks per lane when PIPE is false).
// PIPE: more than NB chunks per lane; two register batches alternate.
constexpr int kGemvMaxM = 4;

template <int KIND, int LK, int NTHR = kThreads>
struct GemvGeom {
  static constexpr int G = kWave / LK;            // lane groups per wave
  static constexpr int UB = (NTHR / kWave) * G;   // units per block
};

// Stage activation rows into LDS: 32 values per (row, chunk), pair-permuted,
// plus each chunk's bias sum 136 * sum(x) taken by the same dot2 chain as the
// main loop (so all-8 codes cancel to an exact zero). Row m comes from
// src + m * K. Within a staged row the 16-byte pieces are ordered by
// (piece v of the chunk, chunk c): lanes that read piece v of consecutive
// chunks touch consecutive 16-byte slots, so a wave's reads are free of bank
// conflicts (chunk-major order put lanes 64 bytes apart, four to a bank group).
// Two (row, chunk) items per thread per pass, both loads issued before use.
// Thread numbering starts at `first` (rotated), so a caller can keep the
// staging off waves that are busy with something else.
struct StageRegs {
  uint4 v[2][4];
};
__device__ __forceinline__ void gemv_stage_load(const uint16_t* __restrict__ src, int nrows, int K,
                                                int i0, StageRegs& r) {
  const int C = K / 32, n = nrows * C, nt = blockDim.x;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = min(i0 + h * nt, n - 1);
    const int m = i / C, c = i - m * C;
    const uint16_t* p = src + static_cast<size_t>(m) * K + c * 32;
#pragma unroll
    for (int v = 0; v < 4; ++v) r.v[h][v] = ld16(p + v * 8);
  }
}
__device__ __forceinline__ void gemv_stage_store(int nrows, int K, int i0, const StageRegs& r,
                                                 uint32_t* xs, float* bsum) {
  const int C = K / 32, n = nrows * C, nt = blockDim.x;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = i0 + h * nt;
    if (i >= n) break;
    const int m = i / C, c = i - m * C;
    float bias = 0.0f;
    uint4* dst = reinterpret_cast<uint4*>(xs + m * (K / 2)) + c;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint4 q = pair_permute(r.v[h][v]);
      bias = dot2_bf16(kBiasPair, q.x, bias);
      bias = dot2_bf16(kBiasPair, q.y, bias);
      bias = dot2_bf16(kBiasPair, q.z, bias);
      bias = dot2_bf16(kBiasPair, q.w, bias);
      dst[v * C] = q;
    }
    bsum[m * C + c] = bias;
  }
}
__device__ __forceinline__ void gemv_stage(const uint16_t* __restrict__ src, int nrows, int K,
                                           uint32_t* xs, float* bsum, int first = 0) {
  const int n = nrows * (K / 32), nt = blockDim.x;
  const int me = (threadIdx.x + nt - first % nt) % nt;
  for (int i0 = me; i0 < n; i0 += 2 * nt) {
    StageRegs r;
    gemv_stage_load(src, nrows, K, i0, r);
    gemv_stage_store(nrows, K, i0, r, xs, bsum);
  }
}

// One 16-byte chunk (32 codes) of two weight rows against MM staged
// activation rows (pair-permuted bf16 in LDS, pieces ordered by (v, chunk); row m
// starts at xrow[m], C chunks per row): raw dot
// products, before the bias sum and the scale. Each code dword is widened once
// (register-held constants: one v_and_or_b32 per pair) and used for all MM
// rows; per row the dot2 chain runs in the same order whatever MM is, so a
// row's result does not depend on how many rows share the codes.
template <int MM>
__device__ __forceinline__ void dot_chunk_rows(const uint4& q0, const uint4& q1,
                                               const uint32_t* const (&xrow)[MM], int c, int C,
                                               const NibbleConsts& nk, float (&d0)[MM],
                                               float (&d1)[MM]) {
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    uint32_t w0 = (&q0.x)[v], w1 = (&q1.x)[v];
    asm volatile("" : "+v"(w0), "+v"(w1));
    uint32_t a0, a1, a2, a3, b0, b1, b2, b3;
    nibble_pairs_r(w0, nk, a0, a1, a2, a3);
    nibble_pairs_r(w1, nk, b0, b1, b2, b3);
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      const uint4 xv = reinterpret_cast<const uint4*>(xrow[m])[v * C + c];
      d0[m] = dot2_bf16(a0, xv.x, d0[m]);
      d0[m] = dot2_bf16(a1, xv.y, d0[m]);
      d0[m] = dot2_bf16(a2, xv.z, d0[m]);
      d0[m] = dot2_bf16(a3, xv.w, d0[m]);
      d1[m] = dot2_bf16(b0, xv.x, d1[m]);
      d1[m] = dot2_bf16(b1, xv.y, d1[m]);
      d1[m] = dot2_bf16(b2, xv.z, d1[m]);
      d1[m] = dot2_bf16(b3, xv.w, d1[m]);
    }
  }
}

// All NB chunks of one lane against MM staged rows (row m at LDS row xr[m]),
// each chunk's partial sums un-biased and scaled, then summed over the LK
// lanes of the group: acc0/acc1 (valid in lane lk == 0) are the two output
// rows' dot products with row m. sc0/sc1 hold each chunk's raw fp16 scale in
// their low 16 bits.
template <int MM, int LK, int NB>
__device__ __forceinline__ void gemv_rows(const uint4 (&q0)[NB], const uint4 (&q1)[NB],
                                          const uint32_t (&sc0)[NB], const uint32_t (&sc1)[NB],
                                          const uint32_t* xs, const float* bsum, int rowlen,
                                          int C, const int (&xr)[MM], int lk,
                                          const NibbleConsts& nk, float (&acc0)[MM],
                                          float (&acc1)[MM]) {
  const uint32_t* xrow[MM];
#pragma unroll
  for (int m = 0; m < MM; ++m) {
    xrow[m] = xs + xr[m] * rowlen;
    acc0[m] = 0.0f;
    acc1[m] = 0.0f;
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int c = lk + b * LK;
    float d0[MM], d1[MM];
#pragma unroll
    for (int m = 0; m < MM; ++m) d0[m] = d1[m] = 0.0f;
    dot_chunk_rows<MM>(q0[b], q1[b], xrow, c, C, nk, d0, d1);
    const float s0 = fp16_bits_to_f32(static_cast<uint16_t>(sc0[b]));
    const float s1 = fp16_bits_to_f32(static_cast<uint16_t>(sc1[b]));
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      const float cs = bsum[xr[m] * C + c];
      acc0[m] += s0 * (d0[m] - cs);
      acc1[m] += s1 * (d1[m] - cs);
    }
  }
#pragma unroll
  for (int m = 0; m < MM; ++m) {
#pragma unroll
    for (int sh = LK / 2; sh >= 1; sh >>= 1) {
      acc0[m] += wave_shfl_xor(acc0[m], sh);
      acc1[m] += wave_shfl_xor(acc1[m], sh);
    }
  }
}

// Runs f(m0, std::integral_constant<int, MM>{}) over the M rows two at a time
// (MM = 2, or 1 for an odd last row), so each pass widens the codes once for
// two rows in straight-line code.
template <typename F>
__device__ __forceinline__ void for_row_pairs(int M, F&& f) {
  for (int m0 = 0; m0 < M; m0 += 2) {
    if (m0 + 1 < M)
      f(m0, std::integral_constant<int, 2>{});
    else
      f(m0, std::integral_constant<int, 1>{});
  }
}

// Per-row result callback: receives the lane-group totals (valid in lane
// lk == 0) of both rows for grouped row p.
struct GemvStore {
  void* out;
  int N;
  template <int KIND>
  __device__ __forceinline__ void put(size_t p, int u, float acc0, float acc1) const {
    if (KIND == 0) {
      static_cast<uint16_t*>(out)[p * (N / 2) + u] = f32_to_bf16(silu_mul(acc0, acc1));
    } else {
      *reinterpret_cast<float2*>(static_cast<float*>(out) + p * N + 2 * u) =
          make_float2(acc0, acc1);
    }
  }
};

// One block's GEMV work for expert e, output tile `tile`, in two steps:
// issue() requests the block's first batch of codes (it needs e and the tile
// only), run() stages what is left and computes.
//   A:    KIND 0: x [T][K] (all T rows are staged, x_staged tells whether the
//         caller already did it); KIND 1: h [R][K] (rows p0.. are staged here).
//   sorted: flat slot of each of the expert's M rows (global or LDS); row m
//   is grouped row p0 + m.
template <int KIND, int LK, int NB, bool PIPE, int NTHR = kThreads>
struct GemvBlock {
  static constexpr int MAXM = kGemvMaxM;
  static constexpr int G = GemvGeom<KIND, LK, NTHR>::G;
  static constexpr int UB = GemvGeom<KIND, LK, NTHR>::UB;
  int C, nch, lk, u;
  bool valid;
  const uint8_t* W0;
  const uint8_t* W1;
  const uint16_t* S0;
  const uint16_t* S1;
  uint4 qa0[NB], qa1[NB], qb0[NB], qb1[NB];
  uint32_t sa[NB], sb[NB];  // raw fp16 scales: low half row 0, high half row 1

  __device__ __forceinline__ GemvBlock(const uint8_t* __restrict__ W,
                                       const uint16_t* __restrict__ S, int e, int tile, int K,
                                       int N) {
    C = K / 32;     // 16-byte code chunks per row
    nch = C / LK;   // chunks per lane (uniform)
    const int units = N / 2;
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x >> 6;
    const int g = lane / LK;
    lk = lane % LK;
    u = tile * UB + wv * G + g;
    valid = u < units;
    const int uc = valid ? u : units - 1;
    const int r0 = (KIND == 0) ? uc : 2 * uc;
    const int r1 = (KIND == 0) ? N / 2 + uc : 2 * uc + 1;
    const size_t rowb = static_cast<size_t>(K / 2), rows = static_cast<size_t>(K / kGroup);
    W0 = W + (static_cast<size_t>(e) * N + r0) * rowb + lk * 16;
    W1 = W + (static_cast<size_t>(e) * N + r1) * rowb + lk * 16;
    S0 = S + (static_cast<size_t>(e) * N + r0) * rows;
    S1 = S + (static_cast<size_t>(e) * N + r1) * rows;
  }
  __device__ __forceinline__ void load_batch(int i0, uint4 (&q0)[NB], uint4 (&q1)[NB],
                                             uint32_t (&sc)[NB]) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int i = PIPE ? min(i0 + b, nch - 1) : b;
      q0[b] = ld16_nt(W0 + i * LK * 16);
      q1[b] = ld16_nt(W1 + i * LK * 16);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int i = PIPE ? min(i0 + b, nch - 1) : b;
      const int c = lk + i * LK;
      sc[b] = static_cast<uint32_t>(S0[c >> 2]) | (static_cast<uint32_t>(S1[c >> 2]) << 16);
    }
  }
  __device__ __forceinline__ void issue() { load_batch(0, qa0, qa1, sa); }

  __device__ __forceinline__ void run(const uint16_t* __restrict__ A, int p0, int M,
                                      const int* sorted, int K, int topk, int T, bool x_staged,
                                      uint32_t* xs, float* bsum, int* tok, const GemvStore& st) {
    const int tid = threadIdx.x;
    if (KIND == 0 && !x_staged) gemv_stage(A, T, K, xs, bsum);

    const NibbleConsts nk = nibble_consts();
    auto finish = [&](float acc0, float acc1, int m) {
#pragma unroll
      for (int sh = LK / 2; sh >= 1; sh >>= 1) {
        acc0 += wave_shfl_xor(acc0, sh);
        acc1 += wave_shfl_xor(acc1, sh);
      }
      if (lk == 0 && valid) st.put<KIND>(static_cast<size_t>(p0 + m), u, acc0, acc1);
    };
    // rows are taken in chunks of MAXM (normally one chunk: M <= T <= 4)
    for (int m0 = 0; m0 < M; m0 += MAXM) {
      const int Mc = min(MAXM, M - m0);
      if (KIND == 0) {
        if (tid < Mc) tok[tid] = sorted[m0 + tid] / topk;
      } else {
        gemv_stage(A + static_cast<size_t>(p0 + m0) * K, Mc, K, xs, bsum);
      }
      __syncthreads();
      if (!PIPE) {
        // all of this lane's codes are in registers: one pass over them for
        // all rows of the chunk
        for_row_pairs(Mc, [&](int mb, auto mm) __attribute__((always_inline)) {
          constexpr int MM = decltype(mm)::value;
          int xr[MM];
#pragma unroll
          for (int m = 0; m < MM; ++m) xr[m] = (KIND == 0) ? tok[mb + m] : mb + m;
          uint32_t s0a[NB], s1a[NB];
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            s0a[b] = sa[b];
            s1a[b] = sa[b] >> 16;
          }
          float acc0[MM], acc1[MM];
          gemv_rows<MM, LK, NB>(qa0, qa1, s0a, s1a, xs, bsum, K / 2, C, xr, lk, nk, acc0, acc1);
          if (lk == 0 && valid) {
#pragma unroll
            for (int m = 0; m < MM; ++m)
              st.put<KIND>(static_cast<size_t>(p0 + m0 + mb + m), u, acc0[m], acc1[m]);
          }
        });
      } else {
        // codes stream through two register batches; rows two at a time, the
        // codes widened once for both
        for (int mp = 0; mp < Mc; mp += 2) {
          const bool two = mp + 1 < Mc;
          const int xr0 = (KIND == 0) ? tok[mp] : mp;
          const int xr1 = two ? ((KIND == 0) ? tok[mp + 1] : mp + 1) : xr0;
          const uint32_t* xrow1[1] = {xs + xr0 * (K / 2)};
          const uint32_t* xrow2[2] = {xs + xr0 * (K / 2), xs + xr1 * (K / 2)};
          float acc[2][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}};
          auto compute_batch = [&](int i0, const uint4 (&q0)[NB], const uint4 (&q1)[NB],
                                   const uint32_t (&sc)[NB]) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
              if (i0 + b < nch) {
                const int c = lk + (i0 + b) * LK;
                const float s0 = fp16_bits_to_f32(static_cast<uint16_t>(sc[b] & 0xFFFFu));
                const float s1 = fp16_bits_to_f32(static_cast<uint16_t>(sc[b] >> 16));
                const float cs0 = bsum[xr0 * C + c];
                if (two) {
                  float d0[2] = {0.0f, 0.0f}, d1[2] = {0.0f, 0.0f};
                  dot_chunk_rows<2>(q0[b], q1[b], xrow2, c, C, nk, d0, d1);
                  const float cs1 = bsum[xr1 * C + c];
                  acc[0][0] += s0 * (d0[0] - cs0);
                  acc[0][1] += s1 * (d1[0] - cs0);
                  acc[1][0] += s0 * (d0[1] - cs1);
                  acc[1][1] += s1 * (d1[1] - cs1);
                } else {
                  float d0[1] = {0.0f}, d1[1] = {0.0f};
                  dot_chunk_rows<1>(q0[b], q1[b], xrow1, c, C, nk, d0, d1);
                  acc[0][0] += s0 * (d0[0] - cs0);
                  acc[0][1] += s1 * (d1[0] - cs0);
                }
              }
            }
          };
          if (m0 != 0 || mp != 0) load_batch(0, qa0, qa1, sa);   // first pass reuses the prefetch
          for (int i0 = 0; i0 < nch; i0 += 2 * NB) {
            if (i0 + NB < nch) load_batch(i0 + NB, qb0, qb1, sb);
            compute_batch(i0, qa0, qa1, sa);
            if (i0 + 2 * NB < nch) load_batch(i0 + 2 * NB, qa0, qa1, sa);
            if (i0 + NB < nch) compute_batch(i0 + NB, qb0, qb1, sb);
          }
          finish(acc[0][0], acc[0][1], m0 + mp);
          if (two) finish(acc[1][0], acc[1][1], m0 + mp + 1);
        }
      }
      __syncthreads();  // tok / LDS rows are rewritten by the next row chunk
    }
  }
};

template <int KIND, int LK, int NB, bool PIPE, int NTHR = kThreads>
__device__ __forceinline__ void gemv_block(const uint16_t* __restrict__ A,
                                           const uint8_t* __restrict__ W,
                                           const uint16_t* __restrict__ S, int e, int tile,
                                           int p0, int M, const int* sorted, int K, int N,
                                           int topk, int T, bool x_staged, uint32_t* xs,
                                           float* bsum, int* tok, const GemvStore& st) {
  GemvBlock<KIND, LK, NB, PIPE, NTHR> b(W, S, e, tile, K, N);
  b.issue();
  b.run(A, p0, M, sorted, K, topk, T, x_staged, xs, bsum, tok, st);
}

// Dynamic LDS of a GEMV block: staged rows (pair-permuted) + bias sums.
inline size_t gemv_lds_bytes(int rows, int K) {
  return static_cast<size_t>(rows) * (K / 2) * 4 + static_cast<size_t>(rows) * (K / 32) * 4;
}

// Stand-alone grouped GEMV (moe_grouped_w4a16_ffn at small T): the expert of
// block slot a comes from the permutation's active list.
template <int KIND, int LK, int NB, bool PIPE>
__global__ __launch_bounds__(kThreads) void w4a16_gemv_kernel(
    const uint16_t* __restrict__ A, const uint8_t* __restrict__ W,
    const uint16_t* __restrict__ S, const int* __restrict__ offsets,
    const int* __restrict__ sorted_slot, const int* __restrict__ active,
    const int* __restrict__ n_active, void* __restrict__ out, int K, int N, int topk,
    int tiles, int T) {
  const int a = blockIdx.x / tiles;
  const int tile = blockIdx.x - a * tiles;
  const int na = *n_active;
  const int e = active[a];  // in bounds: the grid has min(E, R) slots
  if (a >= na) return;      // uniform per block, before any barrier
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  const int rows_staged = (KIND == 0) ? T : kGemvMaxM;
  uint32_t* xs = lds;
  float* bsum = reinterpret_cast<float*>(lds + rows_staged * (K / 2));
  __shared__ int tok[kGemvMaxM];
  const int p0 = offsets[e];
  const int M = offsets[e + 1] - p0;
  gemv_block<KIND, LK, NB, PIPE>(A, W, S, e, tile, p0, M, sorted_slot + p0, K, N, topk, T, false,
                                 xs, bsum, tok, GemvStore{out, N});
}

// ----------------------------------------------------- fused decode layer ----
// Whole layer for T <= 4 in two kernels (moe_layer_w4a16 at small T).
//
// decode_gateup_kernel: block a * tiles + tile serves routed slot a (token
// a / k, pick a % k). Every block routes all T tokens itself (one wave per
// token, the routing of moe_route_topk), so its expert e = ids[a] is known
// right after the top-k and the weight stream starts there; the block of the
// first slot that picked e runs all of e's rows, later slots with the same
// expert exit. Where e's rows sit in grouped order (the stable counting sort
// of moe_permute) follows from wave ballots over the R ids while the codes
// are in flight. The last block writes the routing outputs, the permutation
// and a compact per-expert record {e, p0, M} for the second kernel; it does
// no GEMV work, so that bookkeeping stays off the weight stream's path.
//
// decode_down_kernel: a block owns a tile of NR output rows of H for every
// active expert. Its lane groups walk the (expert, row pair) work items of the
// tile with the next item's codes in flight, read the expert's h rows from
// LDS (all R = T*k grouped rows are staged once) and keep every result in
// LDS, so the block ends holding all k expert outputs of every token for its
// rows: the combine out[t] = sum_j w[t,j] y[t,j] is then taken in increasing
// j inside the block, in the order moe_combine uses. No counters, fences or
// atomics cross blocks.
constexpr int kDecodeMaxT = 4;
constexpr int kDecodeMaxR = kDecodeMaxT * 32;
// Down kernel: 256 blocks (one per CU, so the staged h rows are read once per
// CU), one item in flight per lane group. 1024 threads (four waves per SIMD),
// or 512 when a tile's items all fit one lane group each. Measured against
// two 256-thread blocks per CU with two or four items in flight: 27.1 against
// 37.5 us (decode_large down), 19.55 against 19.81 us per decode_t2 layer;
// 512 threads where the items fit: 17.6 against 17.8 us per decode_t2 layer,
// and 70.3 against 68.6 us per decode_large step where they do not.
constexpr int kDecodeBlocks = 256;
constexpr int kDecodeThreads = 1024;
constexpr int kDecodeSmallThreads = 512;
// Persistent gate/up: 1024 working blocks of 256 threads, four per CU at four
// waves per SIMD (128 VGPRs). Two units in flight per lane group at two waves
// per SIMD (85.0 us per step at H 7168 / E 256), 512-thread blocks (79.4 us)
// and 1024-thread blocks (72.2 us, against 69.0 us) measured slower.
constexpr int kGateupThreads = 256;
constexpr int kDecodeGateupBlocks = 1024;
constexpr int kDecodeSlotMaxBlocks = 2048;   // largest grid of the slot-per-block gate/up
constexpr int kSlotThreads = 256;            // threads per slot-per-block gate/up block (512: slower)

// Routing bookkeeping of the fused layer (the last gate/up block): counts,
// exclusive offsets, active list, stable slot order; writes the routing
// outputs and the per-expert records (entries past n_active repeat the last
// active expert, so readers may index any slot below min(R, E)).
template <int NTHR>
__device__ __forceinline__ void decode_bookkeeping(const int* s_ids, const float* s_w, int* s_off,
                                                   int* s_sorted, int* s_pos, int* s_act,
                                                   int* s_tot, int R, int E, int* ids_out,
                                                   float* w_out, int* offsets_out,
                                                   int* sorted_out, int* pos_out, int* active_out,
                                                   int* n_active_out, int* rec) {
  const int tid = threadIdx.x;
  for (int i = tid; i <= E; i += NTHR) s_off[i] = 0;
  __syncthreads();
  if (tid < R) atomicAdd(&s_off[s_ids[tid]], 1);
  __syncthreads();
  // counts -> exclusive offsets and the active list (E <= 1024: <= 4 per thread)
  const int ept = (E + NTHR - 1) / NTHR;
  int c[4], sc = 0, sf = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * ept + i;
    c[i] = (i < ept && e < E) ? s_off[e] : 0;
    sc += c[i];
    sf += c[i] > 0;
  }
  int tot_c, na;
  int oc = block_excl_scan<NTHR>(sc, s_tot, tot_c);
  int of = block_excl_scan<NTHR>(sf, s_tot, na);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * ept + i;
    if (i < ept && e < E) {
      s_off[e] = oc;
      if (c[i]) s_act[of] = e;
    }
    oc += c[i];
    of += c[i] > 0;
  }
  if (tid == 0) s_off[E] = R;
  __syncthreads();
  // stable position of slot f: its expert's offset + earlier slots of that expert
  if (tid < R) {
    const int id = s_ids[tid];
    int before = 0;
    for (int f = 0; f < tid; ++f) before += (s_ids[f] == id);
    const int p = s_off[id] + before;
    s_sorted[p] = tid;
    s_pos[tid] = p;
  }
  __syncthreads();
  for (int i = tid; i < R; i += NTHR) {
    ids_out[i] = s_ids[i];
    w_out[i] = s_w[i];
    sorted_out[i] = s_sorted[i];
    pos_out[i] = s_pos[i];
  }
  for (int i = tid; i <= E; i += NTHR) offsets_out[i] = s_off[i];
  const int act = R < E ? R : E;
  for (int i = tid; i < act; i += NTHR) {
    const int e = s_act[i < na ? i : na - 1];
    if (i < na) active_out[i] = e;
    rec[1 + 3 * i] = e;
    rec[2 + 3 * i] = s_off[e];
    rec[3 + 3 * i] = s_off[e + 1] - s_off[e];
  }
  if (tid == 0) {
    *n_active_out = na;
    rec[0] = na;
  }
}

// An empty use of loaded registers: the compiler waits for their loads here.
__device__ __forceinline__ void use_regs(const uint4& a, const uint4& b, uint32_t c, uint32_t d) {
  asm volatile("" ::"v"(a.x), "v"(a.y), "v"(a.z), "v"(a.w), "v"(b.x), "v"(b.y), "v"(b.z),
               "v"(b.w), "v"(c), "v"(d));
}

// Slot-per-block gate/up of the fused decode layer, for small grids: block
// a * tiles + tile serves routed slot a (token a / k, pick a % k) and one tile
// of UB units. Its expert e = ids[a] is known right after the top-k, so the
// weight stream starts there; the block of the first slot that picked e runs
// all of e's rows, later slots with the same expert exit. Where e's rows sit
// in grouped order follows from wave ballots over the R ids. The last block
// does the bookkeeping, as in the persistent variant below.
template <int LK, int NB, int S, int NTHR>
__global__ __launch_bounds__(NTHR) void decode_gateup_slot_kernel(
    const float* __restrict__ logits, const uint16_t* __restrict__ x,
    const uint8_t* __restrict__ w13, const uint16_t* __restrict__ s13, int T, int H, int I, int E,
    int k, int tiles, int* __restrict__ ids_out, float* __restrict__ w_out,
    int* __restrict__ offsets_out, int* __restrict__ sorted_out, int* __restrict__ pos_out,
    int* __restrict__ active_out, int* __restrict__ n_active_out, uint16_t* __restrict__ h,
    int* __restrict__ rec) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  uint32_t* xs = lds;                                            // [T][H/2]
  float* bsum = reinterpret_cast<float*>(lds + T * (H / 2));     // [T][H/32]
  int* s_off = reinterpret_cast<int*>(bsum + T * (H / 32));      // [E + 1] (bookkeeping)
  __shared__ int s_ids[kDecodeMaxR];
  __shared__ float s_w[kDecodeMaxR];
  __shared__ int s_sorted[kDecodeMaxR], s_pos[kDecodeMaxR], s_act[kDecodeMaxR];
  __shared__ int s_tot[NTHR / kWave];
  __shared__ int tok[kGemvMaxM];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid >> 6;
  const int R = T * k;

  if (wv < T) wave_topk<S>(logits + static_cast<size_t>(wv) * E, E, k, s_ids + wv * k, s_w + wv * k);
  if (blockIdx.x == gridDim.x - 1) {  // uniform: the bookkeeping block
    __syncthreads();
    decode_bookkeeping<NTHR>(s_ids, s_w, s_off, s_sorted, s_pos, s_act, s_tot, R, E, ids_out,
                                 w_out, offsets_out, sorted_out, pos_out, active_out,
                                 n_active_out, rec);
    return;
  }
  gemv_stage(x, T, H, xs, bsum, T * kWave);  // waves T.. (the top-k waves are busy)
  __syncthreads();
  const int a = blockIdx.x / tiles;
  const int tile = blockIdx.x - a * tiles;
  const int e = s_ids[a];
  // e's rows are the slots f with ids[f] == e, in increasing f; p0 = number of
  // slots with a smaller expert id. Every wave forms the same ballots.
  int p0 = 0, M = 0, earlier = 0;
  for (int f0 = 0; f0 < R; f0 += kWave) {
    const int f = f0 + lane;
    const int id = f < R ? s_ids[f] : E;
    const uint64_t eq = __ballot(id == e);
    p0 += __popcll(__ballot(id < e));
    const uint64_t below = a - f0 >= kWave ? ~0ull : (a - f0 <= 0 ? 0ull : (1ull << (a - f0)) - 1);
    earlier += __popcll(eq & below);
    if (wv == 0 && id == e) s_sorted[M + __popcll(eq & ((1ull << lane) - 1))] = f;
    M += __popcll(eq);
  }
  if (earlier) return;  // uniform: an earlier slot's block runs expert e
  // s_sorted[m] was written by wave 0, the only wave that reads it (tok fill)
  gemv_block<0, LK, NB, false, NTHR>(x, w13, s13, e, tile, p0, M, s_sorted, H, 2 * I, k, T, true, xs,
                               bsum, tok, GemvStore{h, 2 * I});
}

// Persistent gate/up of the fused decode layer. Blocks 0..nblk-1 work, block
// nblk does the bookkeeping. Every block routes the T tokens; each wave then
// lists the active experts in order of first pick (expert, grouped offset,
// rows, their tokens) from the R ids, all waves writing the same table. The
// work is na * I units (an active expert's gate row u with its up row I + u);
// lane group g of the grid takes units g, g + NGt, ..., so every block streams
// an equal share whatever na is.
// LK lanes split the H/32 code chunks of a row, NB = H/32/LK chunks each.
template <int LK, int NB, int S, int NTHR>
__global__ __launch_bounds__(NTHR, 4 * kThreads / NTHR) void decode_gateup_kernel(
    const float* __restrict__ logits, const uint16_t* __restrict__ x,
    const uint8_t* __restrict__ w13, const uint16_t* __restrict__ s13, int T, int H, int I, int E,
    int k, int* __restrict__ ids_out, float* __restrict__ w_out, int* __restrict__ offsets_out,
    int* __restrict__ sorted_out, int* __restrict__ pos_out, int* __restrict__ active_out,
    int* __restrict__ n_active_out, uint16_t* __restrict__ h, int* __restrict__ rec) {
  constexpr int G = kWave / LK;                  // lane groups per wave
  constexpr int NGB = (NTHR / kWave) * G;        // lane groups per block
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  const int C = H / 32;                                          // 16-byte chunks per row
  uint32_t* xs = lds;                                            // [T][H/2]
  float* bsum = reinterpret_cast<float*>(lds + T * (H / 2));     // [T][C]
  int* s_off = reinterpret_cast<int*>(bsum + T * C);             // [E + 1] (bookkeeping)
  __shared__ int s_ids[kDecodeMaxR];
  __shared__ float s_w[kDecodeMaxR];
  __shared__ int s_sorted[kDecodeMaxR], s_pos[kDecodeMaxR], s_act[kDecodeMaxR], s_tot[NTHR / kWave];
  __shared__ int s_ae[kDecodeMaxR], s_ap0[kDecodeMaxR], s_am[kDecodeMaxR];
  __shared__ int s_atok[kDecodeMaxR][kDecodeMaxT];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid >> 6;
  const int R = T * k;
  const int nblk = gridDim.x - 1;

  if (wv < T) wave_topk<S>(logits + static_cast<size_t>(wv) * E, E, k, s_ids + wv * k, s_w + wv * k);
  if (blockIdx.x == nblk) {  // uniform: the bookkeeping block
    __syncthreads();
    decode_bookkeeping<NTHR>(s_ids, s_w, s_off, s_sorted, s_pos, s_act, s_tot, R, E, ids_out,
                                 w_out, offsets_out, sorted_out, pos_out, active_out,
                                 n_active_out, rec);
    return;
  }
  gemv_stage(x, T, H, xs, bsum, T * kWave);  // waves T.. (the top-k waves are busy)
  __syncthreads();

  // active experts in order of first pick; p0 = slots with a smaller id (the
  // expert's first grouped row), tokens in slot order (a token picks an
  // expert at most once, so an expert has at most T rows)
  int na = 0;
  const int id_lo = lane < R ? s_ids[lane] : -1;
  const int id_hi = kWave + lane < R ? s_ids[kWave + lane] : -1;
  for (int f0 = 0; f0 < R; f0 += kWave) {
    const int f = f0 + lane;
    const int id = f0 == 0 ? id_lo : id_hi;
    int lt = 0, before = 0, mm = 0;
    uint32_t toks = 0;  // 2 bits per row: tokens of this expert in slot order
    for (int g = 0; g < R; ++g) {
      const int ig = __builtin_amdgcn_readlane(g < kWave ? id_lo : id_hi, g & (kWave - 1));
      lt += ig < id;
      if (ig == id) {
        before += g < f;
        if (mm < kDecodeMaxT) toks |= static_cast<uint32_t>(g / k) << (2 * mm++);
      }
    }
    const bool first = f < R && before == 0;
    const uint64_t fm = __ballot(first);
    if (first) {
      const int a = na + __popcll(fm & ((1ull << lane) - 1));
      for (int m = 0; m < mm; ++m) s_atok[a][m] = (toks >> (2 * m)) & 3;
      s_ae[a] = id;
      s_ap0[a] = lt;
      s_am[a] = mm;
    }
    na += __popcll(fm);
  }

  const int U = na * I;
  const size_t rowb = static_cast<size_t>(H / 2), srow = static_cast<size_t>(H / kGroup);
  const int gid = blockIdx.x * NGB + wv * G + lane / LK, lk = lane % LK;
  const int NGt = nblk * NGB;
  const NibbleConsts nk = nibble_consts();
  // codes and raw fp16 scales of one unit (a chunk's gate and up scales
  // share one register: the low half the gate row's, the high half the up
  // row's); the scales stay unconverted so that nothing waits on a load until
  // the unit is computed
  struct Unit {
    uint4 q0[NB], q1[NB];
    uint32_t sc[NB];
  };
  Unit ua;
  auto load_unit = [&](int q, Unit& w) {
    q = min(q, U - 1);
    const int a = q / I, u = q - a * I;
    const size_t r0 = static_cast<size_t>(s_ae[a]) * (2 * I) + u;
    const uint8_t* W0 = w13 + r0 * rowb + lk * 16;
    const uint16_t* S0 = s13 + r0 * srow;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      w.q0[b] = ld16_nt(W0 + b * LK * 16);
      w.q1[b] = ld16_nt(W0 + I * rowb + b * LK * 16);
    }
    // chunk c = lk + b * LK has scale group c / 4 = lk / 4 + b * LK / 4: one
    // base address per row and compile-time offsets
    const uint16_t* Sg = S0 + (lk >> 2);
    const uint16_t* Su = Sg + I * srow;
#pragma unroll
    for (int b = 0; b < NB; ++b)
      w.sc[b] = static_cast<uint32_t>(Sg[b * (LK / 4)]) |
                (static_cast<uint32_t>(Su[b * (LK / 4)]) << 16);
  };
  auto run_unit = [&](int q, const Unit& w) __attribute__((always_inline)) {
    // wait for exactly this unit's loads here, in straight-line code, so the
    // row loop below does not drain the other unit's loads as well
#pragma unroll
    for (int b = 0; b < NB; ++b)
      use_regs(w.q0[b], w.q1[b], w.sc[b], w.sc[b]);
    const int a = q / I, u = q - a * I;
    const int p0 = s_ap0[a], M = s_am[a];
    uint32_t s0[NB], s1[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      s0[b] = w.sc[b];
      s1[b] = w.sc[b] >> 16;
    }
    for_row_pairs(M, [&](int mb, auto mm) __attribute__((always_inline)) {
      constexpr int MM = decltype(mm)::value;
      int xr[MM];
#pragma unroll
      for (int m = 0; m < MM; ++m) xr[m] = s_atok[a][mb + m];
      float acc0[MM], acc1[MM];
      gemv_rows<MM, LK, NB>(w.q0, w.q1, s0, s1, xs, bsum, H / 2, C, xr, lk, nk, acc0, acc1);
      if (lk == 0) {
#pragma unroll
        for (int m = 0; m < MM; ++m)
          h[static_cast<size_t>(p0 + mb + m) * I + u] = f32_to_bf16(silu_mul(acc0[m], acc1[m]));
      }
    });
  };
  // units gid, gid + NGt, ...: one unit's codes in flight per lane group; the
  // other waves of the SIMD (four per SIMD) cover its load latency
  for (int q = gid; q < U; q += NGt) {
    load_unit(q, ua);
    run_unit(q, ua);
  }
}

// NB: code chunks per lane (= K / 32 / LK, at most 4 here; larger K uses the
// separate calls). D: work items in flight per lane group. NTHR: block width.
template <int LK, int NB, int D, int NTHR>
__global__ __launch_bounds__(NTHR, NTHR > kThreads ? 4 * kThreads / NTHR : 1) void decode_down_kernel(
    const uint16_t* __restrict__ h, const uint8_t* __restrict__ w2,
    const uint16_t* __restrict__ s2, int T, int H, int I, int E, int k, int upb,
    const int* __restrict__ rec, const int* __restrict__ slot_pos,
    const float* __restrict__ topk_w, float* __restrict__ y, float* __restrict__ out) {
  constexpr int G = kWave / LK;       // lane groups per wave
  constexpr int NG = (NTHR / kWave) * G;   // lane groups per block
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  const int R = T * k;
  const int C = I / 32;
  const int nr = 2 * upb;                                        // rows of H in this tile
  uint32_t* xs = lds;                                            // [R][I/2]
  float* bsum = reinterpret_cast<float*>(lds + R * (I / 2));     // [R][C]
  float* ybuf = bsum + R * C;                                    // [R][nr]
  __shared__ int s_e[kDecodeMaxR], s_p0[kDecodeMaxR], s_m[kDecodeMaxR];
  __shared__ float s_w[kDecodeMaxR];
  __shared__ int s_sp[kDecodeMaxR];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid >> 6;
  const int lg = wv * G + lane / LK, lk = lane % LK;
  const int u0 = blockIdx.x * upb;                 // first unit (row pair) of the tile
  const int units = H / 2;

  // work item q = (active expert a, unit uu of the tile): two W2 rows; codes
  // and raw fp16 scales stay unpacked so nothing waits on a load early
  const size_t rowb = static_cast<size_t>(I / 2), srow = static_cast<size_t>(I / kGroup);
  struct Item {
    uint4 q0[NB], q1[NB];
    uint32_t s0[NB], s1[NB];
  };
  Item it[D];
  auto load_codes = [&](int e, int u, Item& w) {
    const uint8_t* W0 = w2 + (static_cast<size_t>(e) * H + 2 * u) * rowb + lk * 16;
    const uint16_t* S0 = s2 + (static_cast<size_t>(e) * H + 2 * u) * srow;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      w.q0[b] = ld16_nt(W0 + b * LK * 16);
      w.q1[b] = ld16_nt(W0 + rowb + b * LK * 16);
    }
    // chunk c = lk + b * LK has scale group lk / 4 + b * LK / 4
    const uint16_t* Sg = S0 + (lk >> 2);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      w.s0[b] = Sg[b * (LK / 4)];
      w.s1[b] = Sg[srow + b * (LK / 4)];
    }
  };
  // The first D items' codes go out before anything else: their expert is
  // read straight from the record (slot clamped below min(R, E), id clamped to
  // [0, E): every record slot holds a valid expert, the clamps only keep the
  // address in bounds), alongside the count of active experts.
  // the record's expert ids go out first: loads complete in issue order, so
  // the codes that depend on them wait for nothing else; the first pass of h
  // rows follows (it depends on nothing)
  const int act = R < E ? R : E;
  int rec_e[D];
#pragma unroll
  for (int d = 0; d < D; ++d) rec_e[d] = rec[1 + 3 * min((lg + d * NG) / upb, act - 1)];
  const int na = rec[0];
  const int n_stage = R * C;
  StageRegs h0;
  gemv_stage_load(h, R, I, tid, h0);
  // the combine's weights and slot positions were written before this kernel
  // started: request them now, park them in LDS once the h stage has landed
  float my_w = 0.0f;
  int my_sp = 0;
  if (tid < R) {
    my_w = topk_w[tid];
    my_sp = slot_pos[tid];
  }
  // lane groups past the tile's largest item count (min(R, E) experts) have
  // nothing to load
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const int q = lg + d * NG;
    if (q < act * upb)
      load_codes(min(max(rec_e[d], 0), E - 1), min(u0 + (q - (q / upb) * upb), units - 1), it[d]);
  }
  for (int i = tid; i < na; i += NTHR) {
    s_e[i] = rec[1 + 3 * i];
    s_p0[i] = rec[2 + 3 * i];
    s_m[i] = rec[3 + 3 * i];
  }
  gemv_stage_store(R, I, tid, h0, xs, bsum);
  if (tid < R) {
    s_w[tid] = my_w;
    s_sp[tid] = my_sp;
  }
  for (int i0 = tid + 2 * NTHR; i0 < n_stage; i0 += 2 * NTHR) {
    StageRegs r;
    gemv_stage_load(h, R, I, i0, r);
    gemv_stage_store(R, I, i0, r, xs, bsum);
  }
  __syncthreads();
  const int nitems = na * upb;
  const NibbleConsts nk = nibble_consts();
  auto load_item = [&](int q, Item& w) {
    const int qq = min(q, nitems - 1);
    const int a = qq / upb;
    load_codes(s_e[a], min(u0 + (qq - a * upb), units - 1), w);
  };
  auto run_item = [&](int q, const Item& w) __attribute__((always_inline)) {
    // wait for exactly this item's loads here, in straight-line code
#pragma unroll
    for (int b = 0; b < NB; ++b)
      use_regs(w.q0[b], w.q1[b], w.s0[b], w.s1[b]);
    const int a = q / upb;
    const int uu = q - a * upb;
    const int p0 = s_p0[a], M = s_m[a];
    const bool valid = u0 + uu < units;
    for_row_pairs(M, [&](int mb, auto mm) __attribute__((always_inline)) {
      constexpr int MM = decltype(mm)::value;
      int xr[MM];
#pragma unroll
      for (int m = 0; m < MM; ++m) xr[m] = p0 + mb + m;
      float acc0[MM], acc1[MM];
      gemv_rows<MM, LK, NB>(w.q0, w.q1, w.s0, w.s1, xs, bsum, I / 2, C, xr, lk, nk, acc0, acc1);
      if (lk == 0 && valid) {
#pragma unroll
        for (int m = 0; m < MM; ++m) {
          ybuf[xr[m] * nr + 2 * uu] = acc0[m];
          ybuf[xr[m] * nr + 2 * uu + 1] = acc1[m];
          *reinterpret_cast<float2*>(y + static_cast<size_t>(xr[m]) * H + 2 * (u0 + uu)) =
              make_float2(acc0[m], acc1[m]);
        }
      }
    });
  };
  // items lg, lg + NG, ...: D register sets rotate so D - 1 items stream
  // while one is computed (the first D are already in flight)
  for (int q = lg; q < nitems; q += D * NG) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int qq = q + d * NG;
      if (qq < nitems) {
        run_item(qq, it[d]);
        if (qq + D * NG < nitems) load_item(qq + D * NG, it[d]);
      }
    }
  }
  __syncthreads();
  // combine for this tile's rows, in increasing j
  for (int idx = tid; idx < T * nr; idx += NTHR) {
    const int t = idx / nr, r = idx - t * nr;
    const int n = 2 * u0 + r;
    if (n >= H) continue;
    float acc = 0.0f;
    for (int j = 0; j < k; ++j) acc += s_w[t * k + j] * ybuf[s_sp[t * k + j] * nr + r];
    out[static_cast<size_t>(t) * H + n] = acc;
  }
}

template <int KIND, int LK, int NB, bool PIPE>
hipError_t launch_gemv_t(const uint16_t* A, const uint8_t* W, const uint16_t* S,
                         const int* offsets, const int* sorted_slot, const int* active,
                         const int* n_active, void* out, int K, int N, int topk,
                         int max_active, int T, hipStream_t s) {
  constexpr int UB = GemvGeom<KIND, LK>::UB;
  const int units = N / 2;
  const int tiles = (units + UB - 1) / UB;
  const size_t lds = gemv_lds_bytes((KIND == 0) ? T : kGemvMaxM, K);
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&w4a16_gemv_kernel<KIND, LK, NB, PIPE>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((w4a16_gemv_kernel<KIND, LK, NB, PIPE>), dim3(max_active * tiles),
                     dim3(kThreads), lds, s, A, W, S, offsets, sorted_slot, active, n_active,
                     out, K, N, topk, tiles, T);
  return hipGetLastError();
}

// Pick the lane split LK (largest of 16/8/4 dividing the chunk count) and the
// batch shape, then call F<LK, NB, PIPE>::run(args...).
template <template <int, int, bool> class F, typename... Args>
hipError_t gemv_dispatch(int K, Args... args) {
  const int C = K / 32;
  const int LK = (C % 16 == 0 && C >= 64) ? 16 : (C % 8 == 0 ? 8 : 4);
  const int nch = C / LK;
#define MOE_GEMV_NB(LK_)                                          \
  switch (nch) {                                                  \
    case 1: return F<LK_, 1, false>::run(args...);                \
    case 2: return F<LK_, 2, false>::run(args...);                \
    case 3: return F<LK_, 3, false>::run(args...);                \
    case 4: return F<LK_, 4, false>::run(args...);                \
    default: return F<LK_, 4, true>::run(args...);                \
  }
  if (LK == 16) { MOE_GEMV_NB(16) }
  if (LK == 8) { MOE_GEMV_NB(8) }
  MOE_GEMV_NB(4)
#undef MOE_GEMV_NB
}

template <int KIND>
struct GemvLaunch {
  template <int LK, int NB, bool PIPE>
  struct F {
    template <typename... A>
    static hipError_t run(A... a) { return launch_gemv_t<KIND, LK, NB, PIPE>(a...); }
  };
};
template <int LK, int NB, bool PIPE>
using GemvLaunch0 = typename GemvLaunch<0>::template F<LK, NB, PIPE>;
template <int LK, int NB, bool PIPE>
using GemvLaunch1 = typename GemvLaunch<1>::template F<LK, NB, PIPE>;

template <int KIND>
hipError_t launch_gemv(const uint16_t* A, const uint8_t* W, const uint16_t* S,
                       const int* offsets, const int* sorted_slot, const int* active,
                       const int* n_active, void* out, int K, int N, int topk,
                       int max_active, int T, hipStream_t s) {
  if (KIND == 0)
    return gemv_dispatch<GemvLaunch0>(K, A, W, S, offsets, sorted_slot, active, n_active, out, K,
                                      N, topk, max_active, T, s);
  return gemv_dispatch<GemvLaunch1>(K, A, W, S, offsets, sorted_slot, active, n_active, out, K,
                                    N, topk, max_active, T, s);
}

// Lane split of the fused gate/up: an LK in {8, 16, 32} dividing the H/32
// code chunks of a row with at most 4 chunks per lane, else (rows of 256 or
// more chunks) a whole wave per unit with at most 4 chunks per lane, else at
// most 7 (eight chunks of two rows, with their scales, need more than the
// 128 registers of four waves per SIMD); 0 if none. Rows of 64 or more chunks
// take the largest such LK (shorter dot chains per lane: 17.6 -> 17.2 us per
// decode_t2 layer, same-box A/B), shorter rows the smallest (the lane split
// of the stand-alone GEMV there).
inline int decode_gateup_lk(int H) {
  const int C = H / 32;
  if (C >= 256 && C % 64 == 0 && C / 64 <= 4) return 64;
  for (int cap = 4; cap <= 7; cap += 3) {
    if (C >= 64) {
      for (int lk = 32; lk >= 8; lk /= 2)
        if (C % lk == 0 && C / lk <= cap) return lk;
    } else {
      for (int lk = 8; lk <= 32; lk *= 2)
        if (C % lk == 0 && C / lk <= cap) return lk;
    }
  }
  return 0;
}

template <int LK, int NB>
hipError_t launch_decode_gateup_t(const float* logits, const uint16_t* x, const uint8_t* w13,
                                  const uint16_t* s13, int T, int H, int I, int E, int k, int* ids,
                                  float* w, int* offsets, int* sorted_slot, int* slot_pos,
                                  int* active, int* n_active, uint16_t* h, int* rec,
                                  hipStream_t s) {
  const size_t lds = gemv_lds_bytes(T, H) + static_cast<size_t>(E + 1) * 4;
  auto attr = [&](const void* kern) -> hipError_t {
    if (lds <= 64 * 1024) return hipSuccess;
    return hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                               static_cast<int>(lds));
  };
  // slot-per-block while its grid stays within a few blocks per CU (one unit
  // per lane group, all codes in registers); persistent otherwise. Both add
  // the bookkeeping block.
  constexpr int UB = GemvGeom<0, LK, kSlotThreads>::UB;
  const int tiles = (I + UB - 1) / UB;
  const long long slot_blocks = static_cast<long long>(T) * k * tiles;
  if (NB <= 4 && slot_blocks <= kDecodeSlotMaxBlocks) {
    auto go = [&](auto kern) -> hipError_t {
      const hipError_t e = attr(reinterpret_cast<const void*>(kern));
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(slot_blocks) + 1), dim3(kSlotThreads), lds,
                         s, logits, x, w13, s13, T, H, I, E, k, tiles, ids, w, offsets,
                         sorted_slot, slot_pos, active, n_active, h, rec);
      return hipGetLastError();
    };
    constexpr int NBS = NB <= 4 ? NB : 4;
    if (E <= 128) return go(&decode_gateup_slot_kernel<LK, NBS, 2, kSlotThreads>);
    if (E <= 256) return go(&decode_gateup_slot_kernel<LK, NBS, 4, kSlotThreads>);
    return go(&decode_gateup_slot_kernel<LK, NBS, 16, kSlotThreads>);
  }
  auto go = [&](auto kern) -> hipError_t {
    const hipError_t e = attr(reinterpret_cast<const void*>(kern));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(kDecodeGateupBlocks + 1), dim3(kGateupThreads), lds, s, logits, x,
                       w13, s13, T, H, I, E, k, ids, w, offsets, sorted_slot, slot_pos, active,
                       n_active, h, rec);
    return hipGetLastError();
  };
  if (E <= 128) return go(&decode_gateup_kernel<LK, NB, 2, kGateupThreads>);
  if (E <= 256) return go(&decode_gateup_kernel<LK, NB, 4, kGateupThreads>);
  return go(&decode_gateup_kernel<LK, NB, 16, kGateupThreads>);
}

template <int LK, typename... Args>
hipError_t decode_gateup_nb(int nb, Args... args) {
  switch (nb) {
    case 1: return launch_decode_gateup_t<LK, 1>(args...);
    case 2: return launch_decode_gateup_t<LK, 2>(args...);
    case 3: return launch_decode_gateup_t<LK, 3>(args...);
    case 4: return launch_decode_gateup_t<LK, 4>(args...);
    case 5: return launch_decode_gateup_t<LK, 5>(args...);
    case 6: return launch_decode_gateup_t<LK, 6>(args...);
    case 7: return launch_decode_gateup_t<LK, 7>(args...);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_gateup(const float* logits, const uint16_t* x, const uint8_t* w13,
                                const uint16_t* s13, int T, int H, int I, int E, int k, int* ids,
                                float* w, int* offsets, int* sorted_slot, int* slot_pos,
                                int* active, int* n_active, uint16_t* h, int* rec, hipStream_t s) {
  const int lk = decode_gateup_lk(H);
  const int nb = lk ? H / 32 / lk : 0;
  if (lk == 8)
    return decode_gateup_nb<8>(nb, logits, x, w13, s13, T, H, I, E, k, ids, w, offsets,
                               sorted_slot, slot_pos, active, n_active, h, rec, s);
  if (lk == 16)
    return decode_gateup_nb<16>(nb, logits, x, w13, s13, T, H, I, E, k, ids, w, offsets,
                                sorted_slot, slot_pos, active, n_active, h, rec, s);
  if (lk == 32)
    return decode_gateup_nb<32>(nb, logits, x, w13, s13, T, H, I, E, k, ids, w, offsets,
                                sorted_slot, slot_pos, active, n_active, h, rec, s);
  if (lk == 64 && nb == 4)
    return launch_decode_gateup_t<64, 4>(logits, x, w13, s13, T, H, I, E, k, ids, w, offsets,
                                         sorted_slot, slot_pos, active, n_active, h, rec, s);
  return hipErrorInvalidValue;
}

// Down tile size: enough units per block for about `blocks` blocks.
inline int decode_down_upb(int H, int blocks) { return (H / 2 + blocks - 1) / blocks; }

inline size_t decode_down_lds(int T, int H, int I, int k, int upb) {
  const int R = T * k;
  return gemv_lds_bytes(R, I) + static_cast<size_t>(R) * 2 * upb * 4;
}

template <int LK, int NB, bool PIPE>
struct DecodeDownLaunch {
  static hipError_t run(const uint16_t* h, const uint8_t* w2, const uint16_t* s2, int T, int H,
                        int I, int E, int k, const int* rec, const int* slot_pos, const float* w,
                        float* y, float* out, hipStream_t s) {
    if (PIPE) return hipErrorInvalidValue;  // excluded by the host dispatch rule
    const int upb = decode_down_upb(H, kDecodeBlocks);
    const int blocks = (H / 2 + upb - 1) / upb;
    const size_t lds = decode_down_lds(T, H, I, k, upb);
    auto go = [&](auto kern, int nthr) -> hipError_t {
      if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(lds));
        if (e != hipSuccess) return e;
      }
      hipLaunchKernelGGL(kern, dim3(blocks), dim3(nthr), lds, s, h, w2, s2, T, H, I, E, k,
                         upb, rec, slot_pos, w, y, out);
      return hipGetLastError();
    };
    const int act = T * k < E ? T * k : E;
    if (act * upb <= (kDecodeSmallThreads / kWave) * (kWave / LK))
      return go(&decode_down_kernel<LK, (NB < 1 ? 1 : NB), 1, kDecodeSmallThreads>,
                kDecodeSmallThreads);
    return go(&decode_down_kernel<LK, (NB < 1 ? 1 : NB), 1, kDecodeThreads>, kDecodeThreads);
  }
};

// ---------------------------------------------------------------- MFMA ----
// KIND 0: gate/up. Wave w owns h-columns [nt*128 + 32w, +32): B subtile 0 is
//         gate rows, subtile 1 the matching up rows.
// KIND 1: down. Wave w owns W2 rows [nt*256 + 64w, +64) as two subtiles.
// K advances one scale group (128 k) per step with kMfD groups in flight:
// each step requests group g + kMfD - 1 into a register ring of kMfD groups
// per lane (the B codes, 64 contiguous bytes a row, and this thread's share of
// the activation tile), computes group g, then writes group g + 1's
// activations, pair-permuted, into its LDS stage. Computing a group starts by
// moving its codes through the wave's own LDS area into the operand layout. The LDS tile slot L of a stage holds row
// L/16, 16-byte chunk (L%16) ^ (row%16), so the 32 rows an MFMA operand read
// touches land in distinct banks.
// Operand k order: within each 16-k MFMA step s, lane half hf = lane/32 takes
// k = 64*hf + 8*s + {0,4,1,5,2,6,3,7}: B comes out of nibble_pairs() in that
// order and A is stored in it.
// Each group's MFMA partial sums on 128 + q are un-biased by the same MFMA
// chain run on the constant 136 (= 128 + zero point), then scaled: all-8
// codes give exactly zero.
constexpr int kMfD = 3;  // groups in flight

template <int KIND, int MT>
__global__ __launch_bounds__(kThreads, MT == 1 ? 2 : 1) void w4a16_mfma_kernel(
    const uint16_t* __restrict__ A, const uint8_t* __restrict__ W,
    const uint16_t* __restrict__ S, const int* __restrict__ offsets,
    const int* __restrict__ sorted_slot, void* __restrict__ out, int K, int N, int E, int topk,
    int NT) {
  constexpr int BM = 32 * MT;
  constexpr int CPT = BM * 16 / kThreads;   // activation chunks per thread per group
  constexpr int STAGE = BM * 16 * 16;       // bytes of one activation stage
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[kMfD * STAGE];
  // per wave: one group's codes of its two 32-row B subtiles (64 bytes a row)
  __shared__ __attribute__((aligned(16))) uint8_t b_lds[kThreads / kWave][2 * 32 * 64];
  __shared__ int row_src[BM];
  __shared__ int sm_pref[kThreads / kWave];
  __shared__ int sm_out[5];
  extern __shared__ __attribute__((aligned(16))) uint16_t s_lds[];  // [256][G]: fp16 scales of the tile's weight rows

  TileInfo ti;
  if (!find_tile<BM>(offsets, E, NT, sm_pref, sm_out, ti)) return;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int G = K / kGroup;

  // The scales of the tile's 256 weight rows are contiguous runs of S (two
  // 128-row strips, gate and up, or one 256-row strip) starting at multiples
  // of 256 bytes: they are copied to LDS in 16-byte chunks (a per-group load
  // of one fp16 per row would touch 32 rows per instruction). Rows past the
  // expert read as 0 through the buffer resource and are never used. Loads
  // and stores are unconditional (clamped) so all stay in flight together.
  const __amdgpu_buffer_rsrc_t s_rsrc =
      buffer_rsrc(S + static_cast<size_t>(ti.e) * N * G, static_cast<uint32_t>(N * G) * 2u);
  constexpr int kScBatch = 4;
  const int sc_chunks = 32 * G;           // 256 rows * G * 2 bytes / 16
  const uint32_t strip0 = static_cast<uint32_t>((KIND == 0 ? ti.nt * 128 : ti.nt * 256) * G * 2);
  const uint32_t strip1 = static_cast<uint32_t>((N / 2 + ti.nt * 128) * G * 2);
  auto sc_src = [&](int i) -> uint32_t {
    if (KIND == 0 && i >= 16 * G) return strip1 + (i - 16 * G) * 16;
    return strip0 + i * 16;
  };
  uint4 scv[kScBatch];
#pragma unroll
  for (int u = 0; u < kScBatch; ++u)
    scv[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           s_rsrc, sc_src(min(u * kThreads + tid, sc_chunks - 1)), 0, 0));

  // source row of each tile row; rows past the expert's block read the first
  // row (their results are dropped)
  if (tid < BM) {
    const int p = ti.p_begin + tid;
    const int pv = p < ti.p_end ? p : ti.p_begin;
    row_src[tid] = (KIND == 0) ? sorted_slot[pv] / topk : pv;
  }

  // whether this lane's B columns exist (two subtiles)
  bool nvalid[2];
  if (KIND == 0) {
    const int n = ti.nt * 128 + wv * 32 + l32;  // h column
    nvalid[0] = nvalid[1] = n < N / 2;
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) nvalid[j] = ti.nt * 256 + wv * 64 + j * 32 + l32 < N;
  }
  // codes and scales of this expert through buffer resources: per-lane row
  // offsets stay fixed, the group advances a scalar offset
  const uint32_t rowb = static_cast<uint32_t>(K / 2);
  const __amdgpu_buffer_rsrc_t w_rsrc =
      buffer_rsrc(W + static_cast<size_t>(ti.e) * N * rowb, static_cast<uint32_t>(N) * rowb);
  // Codes are fetched row-contiguous: a wave instruction reads 16 rows x 64
  // bytes (four lanes a row, one 16-byte chunk each), rows 0-15 of a subtile
  // in one load and rows 16-31 in the next. Compute moves them through the
  // wave's LDS area into the MFMA operand layout. Rows past the expert read
  // as zeros (or as the up rows, for a gate tile past I); their columns are
  // dropped.
  uint32_t woff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row0 = (KIND == 0) ? j * (N / 2) + ti.nt * 128 + wv * 32 : ti.nt * 256 + wv * 64 + j * 32;
    woff[j] = static_cast<uint32_t>(row0 + (lane >> 2)) * rowb + (lane & 3) * 16;
  }
  // this lane's rows within the tile's 256 scale rows
  int srow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) srow[j] = (KIND == 0) ? j * 128 + wv * 32 + l32 : wv * 64 + j * 32 + l32;
  __syncthreads();
  // scale strips into LDS (read after the main loop's first barrier)
  for (int i0 = 0; i0 < sc_chunks; i0 += kScBatch * kThreads) {
    if (i0 > 0) {
#pragma unroll
      for (int u = 0; u < kScBatch; ++u)
        scv[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                               s_rsrc, sc_src(min(i0 + u * kThreads + tid, sc_chunks - 1)), 0, 0));
    }
#pragma unroll
    for (int u = 0; u < kScBatch; ++u)
      *reinterpret_cast<uint4*>(s_lds + min(i0 + u * kThreads + tid, sc_chunks - 1) * 8) = scv[u];
  }

  // this thread's activation chunks: slot L = tid + 256 v of a stage
  const uint16_t* asrc[CPT];
  int adst[CPT];
#pragma unroll
  for (int v = 0; v < CPT; ++v) {
    const int L = tid + kThreads * v, row = L >> 4, c = (L & 15) ^ (row & 15);
    asrc[v] = A + static_cast<size_t>(row_src[row]) * K + c * 8;
    adst[v] = L * 16;
  }
  // LDS offsets of this lane's A operand for the 8 MFMA steps of a group
  int aoffs[MT][8];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int row = i * 32 + l32;
#pragma unroll
    for (int s = 0; s < 8; ++s) aoffs[i][s] = (row * 16 + ((hf * 8 + s) ^ (row & 15))) * 16;
  }

  struct Grp {
    uint4 q[2][2];
    uint4 a[CPT];
  };
  Grp ring[kMfD];
  auto issue = [&](int g, Grp& b) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      b.q[j][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                w_rsrc, woff[j], g * 64, 0));
      b.q[j][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                w_rsrc, woff[j] + 16 * rowb, g * 64, 0));
    }
#pragma unroll
    for (int v = 0; v < CPT; ++v) b.a[v] = ld16(asrc[v] + g * kGroup);
  };
  auto stage_a = [&](const Grp& b, int stage) {
#pragma unroll
    for (int v = 0; v < CPT; ++v)
      *reinterpret_cast<uint4*>(a_lds + stage * STAGE + adst[v]) = pair_permute(b.a[v]);
  };

  f32x16_t acc[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  const bf16x8_t bias_op =
      __builtin_bit_cast(bf16x8_t, make_uint4(kBiasPair, kBiasPair, kBiasPair, kBiasPair));

  const NibbleConsts nk = nibble_consts();
  auto compute = [&](const Grp& b, int stage, int g) {
    const uint8_t* st = a_lds + stage * STAGE;
    // the group's codes into the operand layout: lane (l32, hf) takes bytes
    // [32 hf, +32) of row l32. Slot (row, chunk c) sits at row * 4 +
    // (c ^ (row / 4 % 4)), so both the writes (16 rows x 4 chunks) and the
    // reads (32 rows, one chunk each) hit distinct banks. The wave's LDS
    // operations complete in order, so no wait or barrier is needed.
    uint8_t* bw = b_lds[wv];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = h * 16 + (lane >> 2), c = lane & 3;
        *reinterpret_cast<uint4*>(bw + j * 2048 + (row * 4 + (c ^ ((row >> 2) & 3))) * 16) = b.q[j][h];
      }
    uint4 bq[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int c = 2 * hf + t;
        bq[j][t] = *reinterpret_cast<const uint4*>(bw + j * 2048 + (l32 * 4 + (c ^ ((l32 >> 2) & 3))) * 16);
      }
    f32x16_t accg[MT][2], cg[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) cg[i][r] = 0.0f;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) accg[i][j][r] = 0.0f;
    }
    // the group's A operands first, so their LDS latency overlaps the MFMAs
    uint4 av[MT][8];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int s = 0; s < 8; ++s) av[i][s] = *reinterpret_cast<const uint4*>(st + aoffs[i][s]);
    uint16_t sc_bits[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) sc_bits[j] = s_lds[srow[j] * G + g];
    __builtin_amdgcn_sched_barrier(0);  // keep them ahead of the unpack and MFMAs
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bf16x8_t bop[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t w = (&bq[j][s >> 2].x)[s & 3];
        uint4 pq;
        nibble_pairs_r(w, nk, pq.x, pq.y, pq.z, pq.w);
        bop[j] = __builtin_bit_cast(bf16x8_t, pq);
      }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const bf16x8_t aop = __builtin_bit_cast(bf16x8_t, av[i][s]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          accg[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop[j], accg[i][j], 0, 0, 0);
        cg[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bias_op, cg[i], 0, 0, 0);
      }
    }
    float bs[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) bs[j] = fp16_bits_to_f32(sc_bits[j]);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] += bs[j] * (accg[i][j][r] - cg[i][r]);
  };

  // Every step requests exactly one group (past the end: the last group
  // again, into a ring slot nothing reads), so the requests stay in a fixed
  // order the compiler's wait counts can follow. Ring slot and LDS stage of
  // group g are both g % kMfD: group g + 1's activations are written while
  // group g's are read, into the stage group g + 1 - kMfD left.
#pragma unroll
  for (int d = 0; d < kMfD - 1; ++d) issue(min(d, G - 1), ring[d]);
  stage_a(ring[0], 0);
  for (int g0 = 0; g0 < G; g0 += kMfD) {
#pragma unroll
    for (int d = 0; d < kMfD; ++d) {
      const int g = g0 + d;
      __syncthreads();  // group g's stage is written; group g + 1's is free
      issue(min(g + kMfD - 1, G - 1), ring[(d + kMfD - 1) % kMfD]);
      if (g < G) compute(ring[d], d, g);
      if (g + 1 < G) stage_a(ring[(d + 1) % kMfD], (d + 1) % kMfD);
    }
  }

  // epilogue: C layout of 32x32 MFMA: lane holds column l32, rows
  // 8*(r/4) + 4*hf + (r%4), r = 0..15. Stores go through a buffer resource
  // based at the tile's first row and column, at 32-bit offsets: rows past the
  // expert's block lie past the resource's end, columns past the row width are
  // sent there, and the hardware drops both (no branch per element).
  constexpr uint32_t kPastEnd = 0x80000000u;
  constexpr uint32_t esz = (KIND == 0) ? 2 : 4;   // bf16 h or float32 y
  const int ow = (KIND == 0) ? N / 2 : N;
  const int cb = (KIND == 0) ? ti.nt * 128 : ti.nt * 256;
  const int rows = min(ti.p_end - ti.p_begin, BM);
  const uint32_t orowb = static_cast<uint32_t>(ow) * esz;
  const __amdgpu_buffer_rsrc_t o_rsrc = buffer_rsrc(
      static_cast<char*>(out) + (static_cast<size_t>(ti.p_begin) * ow + cb) * esz,
      static_cast<uint32_t>(rows - 1) * orowb + static_cast<uint32_t>(ow - cb) * esz);
  uint32_t coff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = (KIND == 0) ? wv * 32 + l32 : wv * 64 + j * 32 + l32;
    coff[j] = nvalid[j] ? static_cast<uint32_t>(hf * 4) * orowb + c * esz : kPastEnd;
  }
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t roff = static_cast<uint32_t>(i * 32 + (r >> 2) * 8 + (r & 3)) * orowb;
      if (KIND == 0) {
        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(silu_mul(acc[i][0][r], acc[i][1][r])),
                                              o_rsrc, coff[0] + roff, 0, 0);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          // through a scalar: a bit cast of the vector element itself read
          // element 0 for every r (clang)
          const float v = acc[i][j][r];
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), o_rsrc,
                                                coff[j] + roff, 0, 0);
        }
      }
    }
  }
}

template <int KIND, int MT>
hipError_t launch_mfma_t(const uint16_t* A, const uint8_t* W, const uint16_t* S,
                         const int* offsets, const int* sorted_slot, void* out, int K, int N,
                         int E, int topk, int T, hipStream_t s) {
  constexpr int BM = 32 * MT;
  const int NT = (KIND == 0) ? (N / 2 + 127) / 128 : (N + 255) / 256;
  const long long R = static_cast<long long>(T) * topk;
  const long long act = R < E ? R : E;
  // upper bound of m-tiles: sum over active experts of ceil(rows / BM)
  const long long mt_up = (R + BM - 1) / BM + act;
  long long grid = mt_up * NT;
  grid = (grid + 7) / 8 * 8;
  const size_t lds = static_cast<size_t>(256) * (K / kGroup) * 2;   // the tile's scale strips
  hipLaunchKernelGGL((w4a16_mfma_kernel<KIND, MT>), dim3(static_cast<unsigned>(grid)),
                     dim3(kThreads), lds, s, A, W, S, offsets, sorted_slot, out, K, N, E, topk, NT);
  return hipGetLastError();
}

}  // namespace

bool w4a16_uses_gemv(int T, int, int, int, int) { return T <= kGemvMaxT; }

size_t w4a16_workspace_bytes(int T, int, int I, int, int k) {
  return align_up(static_cast<size_t>(T) * k * I * sizeof(uint16_t), 256);
}

hipError_t launch_w4a16_ffn(int T, int H, int I, int E, int k, const uint16_t* x,
                            const uint8_t* w13, const uint16_t* s13, const uint8_t* w2,
                            const uint16_t* s2, const int* offsets, const int* sorted_slot,
                            const int* active, const int* n_active, float* y, void* ws,
                            hipStream_t s) {
  if (T == 0) return hipSuccess;
  uint16_t* h = static_cast<uint16_t*>(ws);
  const int R = T * k;
  const int max_active = R < E ? R : E;
  hipError_t err;
  if (T <= kGemvMaxT) {
    err = launch_gemv<0>(x, w13, s13, offsets, sorted_slot, active, n_active, h, H, 2 * I, k,
                         max_active, T, s);
    if (err != hipSuccess) return err;
    return launch_gemv<1>(h, w2, s2, offsets, sorted_slot, active, n_active, y, I, H, k,
                          max_active, T, s);
  }
  const double avg_rows = static_cast<double>(R) / max_active;
  if (avg_rows <= 48.0) {
    err = launch_mfma_t<0, 1>(x, w13, s13, offsets, sorted_slot, h, H, 2 * I, E, k, T, s);
    if (err != hipSuccess) return err;
    return launch_mfma_t<1, 1>(h, w2, s2, offsets, sorted_slot, y, I, H, E, k, T, s);
  }
  err = launch_mfma_t<0, 2>(x, w13, s13, offsets, sorted_slot, h, H, 2 * I, E, k, T, s);
  if (err != hipSuccess) return err;
  return launch_mfma_t<1, 2>(h, w2, s2, offsets, sorted_slot, y, I, H, E, k, T, s);
}

// ------------------------------------------------------------ whole layer ----
namespace {
struct LayerWs {
  uint16_t* h;
  int* rec;
  void* perm;
};
LayerWs layer_carve(void* ws, int T, int I, int E, int k) {
  const size_t R = static_cast<size_t>(T) * k;
  const size_t act = R < static_cast<size_t>(E) ? R : static_cast<size_t>(E);
  char* p = static_cast<char*>(ws);
  LayerWs w;
  w.h = reinterpret_cast<uint16_t*>(p);
  p += align_up(R * I * sizeof(uint16_t), 256);
  w.rec = reinterpret_cast<int*>(p);
  p += align_up((1 + 3 * act) * sizeof(int), 256);
  w.perm = p;
  return w;
}
// The two-kernel decode layer: T <= 4, the down kernel's codes fit one
// register batch (I / 32 / LK <= 4) and its staged h rows fit LDS.
bool layer_fused(int T, int H, int I, int k) {
  if (T > kDecodeMaxT || T * k > kDecodeMaxR || decode_gateup_lk(H) == 0) return false;
  const int C = I / 32;
  const int LK = (C % 16 == 0 && C >= 64) ? 16 : (C % 8 == 0 ? 8 : 4);
  if (C / LK > 4) return false;
  return decode_down_lds(T, H, I, k, decode_down_upb(H, kDecodeBlocks)) <= 150 * 1024;
}
}  // namespace

size_t w4a16_layer_workspace_bytes(int T, int, int I, int E, int k) {
  const size_t R = static_cast<size_t>(T) * k;
  const size_t act = R < static_cast<size_t>(E) ? R : static_cast<size_t>(E);
  return align_up(R * I * sizeof(uint16_t), 256) + align_up((1 + 3 * act) * sizeof(int), 256) +
         align_up(permute_workspace_bytes(T, E, k), 256);
}

hipError_t launch_w4a16_layer(int T, int H, int I, int E, int k, const float* logits,
                              const uint16_t* x, const uint8_t* w13, const uint16_t* s13,
                              const uint8_t* w2, const uint16_t* s2, int* ids, float* w,
                              int* offsets, int* sorted_slot, int* slot_pos, int* active,
                              int* n_active, float* y, float* out, void* ws, hipStream_t s) {
  const LayerWs lw = layer_carve(ws, T, I, E, k);
  if (T > 0 && layer_fused(T, H, I, k)) {
    hipError_t err = launch_decode_gateup(logits, x, w13, s13, T, H, I, E, k, ids, w, offsets,
                                          sorted_slot, slot_pos, active, n_active, lw.h, lw.rec,
                                          s);
    if (err != hipSuccess) return err;
    return gemv_dispatch<DecodeDownLaunch>(I, lw.h, w2, s2, T, H, I, E, k, lw.rec, slot_pos, w,
                                           y, out, s);
  }
  hipError_t err = launch_route_topk(logits, T, E, k, ids, w, s);
  if (err != hipSuccess) return err;
  err = launch_permute(ids, T, E, k, offsets, sorted_slot, slot_pos, active, n_active, lw.perm, s);
  if (err != hipSuccess) return err;
  err = launch_w4a16_ffn(T, H, I, E, k, x, w13, s13, w2, s2, offsets, sorted_slot, active,
                         n_active, y, lw.h, s);
  if (err != hipSuccess) return err;
  return launch_combine(y, slot_pos, w, T, H, k, out, s);
}

}  // namespace moe
