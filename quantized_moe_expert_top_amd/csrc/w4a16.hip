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
#include "common.h"
#include "launch.h"
#include "tiles.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kGemvMaxT = 4;

// ---------------------------------------------------------------- GEMV ----
// KIND 0: gate/up (A = x rows of the tokens, out = h bf16 [R, I]).
// KIND 1: down    (A = h rows of the expert's block, out = y float32 [R, N]).
// A block owns one routed expert (active slot blockIdx / tiles) and UB units
// of output (a unit is a gate row with its up row, or two down rows). Inside
// a wave, LK lanes split K: lane lk reads the 16-byte code chunks lk, lk+LK,
// ... of each of its two rows (coalesced LK*16-byte runs), so per chunk the
// 64 bytes of activations it needs are read from LDS once for both rows.
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

template <int KIND, int LK, int NB, bool PIPE>
__global__ __launch_bounds__(kThreads) void w4a16_gemv_kernel(
    const uint16_t* __restrict__ A, const uint8_t* __restrict__ W,
    const uint16_t* __restrict__ S, const int* __restrict__ offsets,
    const int* __restrict__ sorted_slot, const int* __restrict__ active,
    const int* __restrict__ n_active, void* __restrict__ out, int K, int N, int topk,
    int tiles, int T) {
  constexpr int MAXM = kGemvMaxM;
  constexpr int G = kWave / LK;               // lane groups per wave
  constexpr int UB = (kThreads / kWave) * G;  // units per block
  const int a = blockIdx.x / tiles;
  const int tile = blockIdx.x - a * tiles;
  const int na = *n_active;
  const int e_raw = active[a];  // in bounds: grid has min(E, R) slots
  if (a >= na) return;          // uniform per block, before any barrier
  const int e = e_raw;
  const int C = K / 32;         // 16-byte code chunks per row
  const int nch = C / LK;       // chunks per lane (uniform)
  const int units = N / 2;

  extern __shared__ uint32_t lds[];
  const int rows_staged = (KIND == 0) ? T : MAXM;
  uint32_t* xs = lds;                                                  // [rows][K/2]
  float* bsum = reinterpret_cast<float*>(lds + rows_staged * (K / 2));  // [rows][C]
  __shared__ int tok[MAXM];

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid >> 6;
  const int g = lane / LK, lk = lane % LK;
  const int u = tile * UB + wv * G + g;
  const bool valid = u < units;
  const int uc = valid ? u : units - 1;
  const int r0 = (KIND == 0) ? uc : 2 * uc;
  const int r1 = (KIND == 0) ? N / 2 + uc : 2 * uc + 1;
  const size_t rowb = static_cast<size_t>(K / 2), rows = static_cast<size_t>(K / kGroup);
  const uint8_t* W0 = W + (static_cast<size_t>(e) * N + r0) * rowb + lk * 16;
  const uint8_t* W1 = W + (static_cast<size_t>(e) * N + r1) * rowb + lk * 16;
  const uint16_t* S0 = S + (static_cast<size_t>(e) * N + r0) * rows;
  const uint16_t* S1 = S + (static_cast<size_t>(e) * N + r1) * rows;

  uint4 qa0[NB], qa1[NB], qb0[NB], qb1[NB];
  uint32_t sa[NB], sb[NB];  // raw fp16 scales: low half row 0, high half row 1
  auto load_batch = [&](int i0, uint4 (&q0)[NB], uint4 (&q1)[NB], uint32_t (&sc)[NB]) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int i = PIPE ? min(i0 + b, nch - 1) : b;
      q0[b] = ld16(W0 + i * LK * 16);
      q1[b] = ld16(W1 + i * LK * 16);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int i = PIPE ? min(i0 + b, nch - 1) : b;
      const int c = lk + i * LK;
      sc[b] = static_cast<uint32_t>(S0[c >> 2]) | (static_cast<uint32_t>(S1[c >> 2]) << 16);
    }
  };
  load_batch(0, qa0, qa1, sa);

  const int p0 = offsets[e];
  const int M = offsets[e + 1] - p0;

  // stage activation rows: 32 values per (row, chunk), pair-permuted, plus the
  // chunk's bias sum 136 * sum(x) taken by the same dot2 chain as the main loop
  // (so all-8 codes cancel to an exact zero)
  auto stage = [&](int nrows, int m0) {
    for (int i = tid; i < nrows * C; i += kThreads) {
      const int m = i / C, c = i - m * C;
      const uint16_t* src = (KIND == 0) ? A + static_cast<size_t>(m) * K + c * 32
                                        : A + static_cast<size_t>(p0 + m0 + m) * K + c * 32;
      uint4 xv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) xv[v] = ld16(src + v * 8);
      float bias = 0.0f;
      uint4* dst = reinterpret_cast<uint4*>(xs + m * (K / 2) + c * 16);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint4 p = pair_permute(xv[v]);
        bias = dot2_bf16(kBiasPair, p.x, bias);
        bias = dot2_bf16(kBiasPair, p.y, bias);
        bias = dot2_bf16(kBiasPair, p.z, bias);
        bias = dot2_bf16(kBiasPair, p.w, bias);
        dst[v] = p;
      }
      bsum[m * C + c] = bias;
    }
  };
  if (KIND == 0) stage(T, 0);

  // one 16-byte chunk (32 codes) of both rows against one staged activation row
  auto dot_chunk = [&](const uint4& q0, const uint4& q1, int xr, int c, float& d0, float& d1) {
    const uint4* xp = reinterpret_cast<const uint4*>(xs + xr * (K / 2) + c * 16);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint4 xv = xp[v];
      uint32_t w0 = (&q0.x)[v], w1 = (&q1.x)[v];
      // keep the widening inside the row loop: hoisting it would hold 4x the
      // code registers live for every row pass, and most experts see one row
      asm volatile("" : "+v"(w0), "+v"(w1));
      uint32_t a0, a1, a2, a3;
      nibble_pairs(w0, a0, a1, a2, a3);
      d0 = dot2_bf16(a0, xv.x, d0);
      d0 = dot2_bf16(a1, xv.y, d0);
      d0 = dot2_bf16(a2, xv.z, d0);
      d0 = dot2_bf16(a3, xv.w, d0);
      nibble_pairs(w1, a0, a1, a2, a3);
      d1 = dot2_bf16(a0, xv.x, d1);
      d1 = dot2_bf16(a1, xv.y, d1);
      d1 = dot2_bf16(a2, xv.z, d1);
      d1 = dot2_bf16(a3, xv.w, d1);
    }
  };
  auto finish = [&](float acc0, float acc1, int m) {
#pragma unroll
    for (int sh = LK / 2; sh >= 1; sh >>= 1) {
      acc0 += wave_shfl_xor(acc0, sh);
      acc1 += wave_shfl_xor(acc1, sh);
    }
    if (lk == 0 && valid) {
      const size_t p = static_cast<size_t>(p0 + m);
      if (KIND == 0) {
        static_cast<uint16_t*>(out)[p * (N / 2) + u] = f32_to_bf16(silu_mul(acc0, acc1));
      } else {
        *reinterpret_cast<float2*>(static_cast<float*>(out) + p * N + 2 * u) =
            make_float2(acc0, acc1);
      }
    }
  };

  // rows are taken in chunks of MAXM (normally one chunk: M <= T <= 4)
  for (int m0 = 0; m0 < M; m0 += MAXM) {
    const int Mc = min(MAXM, M - m0);
    if (KIND == 0) {
      if (tid < Mc) tok[tid] = sorted_slot[p0 + m0 + tid] / topk;
    } else {
      stage(Mc, m0);
    }
    __syncthreads();
    if (!PIPE) {
      // all of this lane's codes are in registers: one pass per row
      for (int m = 0; m < Mc; ++m) {
        const int xr = (KIND == 0) ? tok[m] : m;
        float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int c = lk + b * LK;
          float d0 = 0.0f, d1 = 0.0f;
          dot_chunk(qa0[b], qa1[b], xr, c, d0, d1);
          const float cs = bsum[xr * C + c];
          acc0 += fp16_bits_to_f32(static_cast<uint16_t>(sa[b] & 0xFFFFu)) * (d0 - cs);
          acc1 += fp16_bits_to_f32(static_cast<uint16_t>(sa[b] >> 16)) * (d1 - cs);
        }
        finish(acc0, acc1, m0 + m);
      }
    } else {
      // codes stream through two register batches; rows two at a time
      for (int mp = 0; mp < Mc; mp += 2) {
        const bool two = mp + 1 < Mc;
        const int xr0 = (KIND == 0) ? tok[mp] : mp;
        const int xr1 = two ? ((KIND == 0) ? tok[mp + 1] : mp + 1) : xr0;
        float acc[2][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}};
        auto compute_batch = [&](int i0, const uint4 (&q0)[NB], const uint4 (&q1)[NB],
                                 const uint32_t (&sc)[NB]) {
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            if (i0 + b < nch) {
              const int c = lk + (i0 + b) * LK;
              const float s0 = fp16_bits_to_f32(static_cast<uint16_t>(sc[b] & 0xFFFFu));
              const float s1 = fp16_bits_to_f32(static_cast<uint16_t>(sc[b] >> 16));
              float d0 = 0.0f, d1 = 0.0f;
              dot_chunk(q0[b], q1[b], xr0, c, d0, d1);
              const float cs0 = bsum[xr0 * C + c];
              acc[0][0] += s0 * (d0 - cs0);
              acc[0][1] += s1 * (d1 - cs0);
              if (two) {
                float e0 = 0.0f, e1 = 0.0f;
                dot_chunk(q0[b], q1[b], xr1, c, e0, e1);
                const float cs1 = bsum[xr1 * C + c];
                acc[1][0] += s0 * (e0 - cs1);
                acc[1][1] += s1 * (e1 - cs1);
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

template <int KIND, int LK, int NB, bool PIPE>
hipError_t launch_gemv_t(const uint16_t* A, const uint8_t* W, const uint16_t* S,
                         const int* offsets, const int* sorted_slot, const int* active,
                         const int* n_active, void* out, int K, int N, int topk,
                         int max_active, int T, hipStream_t s) {
  constexpr int UB = (kThreads / kWave) * (kWave / LK);
  const int units = N / 2;
  const int tiles = (units + UB - 1) / UB;
  const int rows_staged = (KIND == 0) ? T : kGemvMaxM;
  const size_t lds = static_cast<size_t>(rows_staged) * (K / 2) * 4 +
                     static_cast<size_t>(rows_staged) * (K / 32) * 4;
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

template <int KIND, int LK>
hipError_t launch_gemv_lk(const uint16_t* A, const uint8_t* W, const uint16_t* S,
                          const int* offsets, const int* sorted_slot, const int* active,
                          const int* n_active, void* out, int K, int N, int topk,
                          int max_active, int T, hipStream_t s) {
  const int nch = K / 32 / LK;
#define MOE_GEMV_CASE(NB_, PIPE_)                                                              \
  return launch_gemv_t<KIND, LK, NB_, PIPE_>(A, W, S, offsets, sorted_slot, active, n_active, \
                                             out, K, N, topk, max_active, T, s)
  switch (nch) {
    case 1: MOE_GEMV_CASE(1, false);
    case 2: MOE_GEMV_CASE(2, false);
    case 3: MOE_GEMV_CASE(3, false);
    case 4: MOE_GEMV_CASE(4, false);
    default: MOE_GEMV_CASE(4, true);
  }
#undef MOE_GEMV_CASE
}

template <int KIND>
hipError_t launch_gemv(const uint16_t* A, const uint8_t* W, const uint16_t* S,
                       const int* offsets, const int* sorted_slot, const int* active,
                       const int* n_active, void* out, int K, int N, int topk,
                       int max_active, int T, hipStream_t s) {
  const int C = K / 32;
  if (C % 16 == 0 && C >= 64)
    return launch_gemv_lk<KIND, 16>(A, W, S, offsets, sorted_slot, active, n_active, out, K, N,
                                    topk, max_active, T, s);
  if (C % 8 == 0)
    return launch_gemv_lk<KIND, 8>(A, W, S, offsets, sorted_slot, active, n_active, out, K, N,
                                   topk, max_active, T, s);
  return launch_gemv_lk<KIND, 4>(A, W, S, offsets, sorted_slot, active, n_active, out, K, N,
                                 topk, max_active, T, s);
}

// ---------------------------------------------------------------- MFMA ----
constexpr int kALd = kGroup + 8;  // LDS row stride of the activation tile (bf16)

// KIND 0: gate/up. Wave w owns h-columns [nt*128 + 32w, +32): B subtile 0 is
//         gate rows, subtile 1 the matching up rows.
// KIND 1: down. Wave w owns W2 rows [nt*256 + 64w, +64) as two subtiles.
// Operand k order: within each 16-k MFMA step, lane half hf = lane/32 takes
// k = 64*hf + 8*s + {0,4,1,5,2,6,3,7} (s = step); A is stored in LDS in that
// pair order, B comes out of nibble_pairs() in it.
template <int KIND, int MT>
__global__ __launch_bounds__(kThreads) void w4a16_mfma_kernel(
    const uint16_t* __restrict__ A, const uint8_t* __restrict__ W,
    const uint16_t* __restrict__ S, const int* __restrict__ offsets,
    const int* __restrict__ sorted_slot, void* __restrict__ out, int K, int N, int E,
    int topk, int NT) {
  constexpr int BM = 32 * MT;
  constexpr int CPT = BM * 16 / kThreads;  // 16-byte A chunks per thread per group
  __shared__ __attribute__((aligned(16))) uint16_t a_lds[2][BM * kALd];
  __shared__ int sm_pref[kThreads / kWave];
  __shared__ int sm_out[3];

  TileInfo ti;
  if (!find_tile<BM>(offsets, E, NT, sm_pref, sm_out, ti)) return;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int G = K / kGroup;
  const size_t rowb = static_cast<size_t>(K / 2);

  // B rows of this lane (two subtiles)
  int nrow[2];
  bool nvalid[2];
  if (KIND == 0) {
    const int n = ti.nt * 128 + wv * 32 + l32;  // h column
    nvalid[0] = nvalid[1] = n < N / 2;
    const int nc = nvalid[0] ? n : N / 2 - 1;
    nrow[0] = nc;
    nrow[1] = N / 2 + nc;
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = ti.nt * 256 + wv * 64 + j * 32 + l32;
      nvalid[j] = n < N;
      nrow[j] = nvalid[j] ? n : N - 1;
    }
  }
  const uint8_t* Wr[2];
  const uint16_t* Sr[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    Wr[j] = W + (static_cast<size_t>(ti.e) * N + nrow[j]) * rowb + hf * 32;
    Sr[j] = S + (static_cast<size_t>(ti.e) * N + nrow[j]) * G;
  }

  // A rows staged by this thread: chunk q = tid + 256*v -> row q/16, chunk q%16
  const uint16_t* arow[CPT];
#pragma unroll
  for (int v = 0; v < CPT; ++v) {
    const int q = tid + kThreads * v;
    const int r = q >> 4, ch = q & 15;
    const int p = ti.p_begin + r;
    if (p < ti.p_end) {
      const size_t src = (KIND == 0) ? static_cast<size_t>(sorted_slot[p] / topk) : static_cast<size_t>(p);
      arow[v] = A + src * K + ch * 8;
    } else {
      arow[v] = nullptr;
    }
  }

  auto load_a = [&](int g, uint4* regs) {
#pragma unroll
    for (int v = 0; v < CPT; ++v)
      regs[v] = arow[v] ? ld16(arow[v] + g * kGroup) : make_uint4(0, 0, 0, 0);
  };
  auto store_a = [&](int buf, const uint4* regs) {
#pragma unroll
    for (int v = 0; v < CPT; ++v) {
      const int q = tid + kThreads * v;
      const int r = q >> 4, ch = q & 15;
      *reinterpret_cast<uint4*>(&a_lds[buf][r * kALd + ch * 8]) = pair_permute(regs[v]);
    }
  };
  auto load_b = [&](int g, uint4 (&bq)[2][2], float (&bs)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      bq[j][0] = ld16(Wr[j] + g * 64);
      bq[j][1] = ld16(Wr[j] + g * 64 + 16);
      bs[j] = fp16_bits_to_f32(Sr[j][g]);
    }
  };

  f32x16_t acc[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  uint4 areg[CPT];
  uint4 bq[2][2], bq_next[2][2];
  float bs[2], bs_next[2];
  load_a(0, areg);
  store_a(0, areg);
  load_b(0, bq, bs);
  __syncthreads();

  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    const bool more = g + 1 < G;
    if (more) {
      load_a(g + 1, areg);
      load_b(g + 1, bq_next, bs_next);
    }
    // accg: the group's partial sums on 128 + q; cg: the same MFMA chain on
    // constant 136 (= 128 + zero point), i.e. its exact bias term
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
    const bf16x8_t bias_op = __builtin_bit_cast(
        bf16x8_t, make_uint4(kBiasPair, kBiasPair, kBiasPair, kBiasPair));
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bf16x8_t bop[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t w = (&bq[j][s >> 2].x)[s & 3];
        uint4 p;
        nibble_pairs(w, p.x, p.y, p.z, p.w);
        bop[j] = __builtin_bit_cast(bf16x8_t, p);
      }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const uint4 av = *reinterpret_cast<const uint4*>(
            &a_lds[buf][(i * 32 + l32) * kALd + hf * 64 + s * 8]);
        const bf16x8_t aop = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          accg[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop[j], accg[i][j], 0, 0, 0);
        cg[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bias_op, cg[i], 0, 0, 0);
      }
    }
    // un-bias and scale the group's partial sums
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] += bs[j] * (accg[i][j][r] - cg[i][r]);
    if (more) {
      store_a(buf ^ 1, areg);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bq[j][0] = bq_next[j][0];
        bq[j][1] = bq_next[j][1];
        bs[j] = bs_next[j];
      }
    }
    __syncthreads();
  }

  // epilogue: C layout of 32x32 MFMA: lane holds column l32, rows
  // 8*(r/4) + 4*hf + (r%4), r = 0..15
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = i * 32 + (r >> 2) * 8 + hf * 4 + (r & 3);
      const int p = ti.p_begin + m;
      if (p >= ti.p_end) continue;
      if (KIND == 0) {
        if (nvalid[0]) {
          const int n = ti.nt * 128 + wv * 32 + l32;
          static_cast<uint16_t*>(out)[static_cast<size_t>(p) * (N / 2) + n] =
              f32_to_bf16(silu_mul(acc[i][0][r], acc[i][1][r]));
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (nvalid[j])
            static_cast<float*>(out)[static_cast<size_t>(p) * N + nrow[j]] = acc[i][j][r];
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
  hipLaunchKernelGGL((w4a16_mfma_kernel<KIND, MT>), dim3(static_cast<unsigned>(grid)),
                     dim3(kThreads), 0, s, A, W, S, offsets, sorted_slot, out, K, N, E, topk, NT);
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

}  // namespace moe
