// Grouped SwiGLU expert FFN, W4A8: int4 g128 weights (the W4A16 storage)
// against per-token int8 activations, on int8 MFMA.
//
// "Measured results", section "Speed": W4A8 beside W4A16 as a weight path.
//   1. quant: per row, s = absmax/127 (IEEE float32 division), codes
//      rint(x/s) clamped to [-127, 127]; also the sum of each 128-wide group
//      of codes (for the zero point).
//   2. gate/up: v_mfma_i32_32x32x32_i8 over (expert, 32-row, 128 h-column)
//      tiles. Codes 0..15 are unpacked to int8 as stored; per 128-k group the
//      exact integer dot is corrected by 8 * (group code sum), scaled by the
//      group's fp16 scale and accumulated in float32; the epilogue applies the
//      row scale and SwiGLU, writing h float32 in grouped order.
//   3. h quant: step 1 on h, one row per routed slot.
//   4. down: step 2 on hq against W2; y = hs * acc, float32.
#include "common.h"
#include "launch.h"
#include "tiles.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kBM = 32;     // rows per tile
constexpr int kD = 3;       // 128-k groups in flight

// --------------------------------------------------------- quantization ----
__device__ __forceinline__ int quant_code4a8(float v, float s) {
  if (s == 0.0f) return 0;
  float q = rintf(v / s);
  q = fminf(fmaxf(q, -127.0f), 127.0f);
  return static_cast<int>(q);
}

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&v)[8]) {
  const uint4 w = ld16(p);
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16lo(u[i]);
    v[2 * i + 1] = bf16hi(u[i]);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// One wave per row of K values (bf16 x rows or float32 h rows), K % 128 == 0.
// Lane l takes 8-value chunks l, l + 64, ...; a 128-wide group is 16 chunks,
// i.e. one 16-lane row of the wave, so its code sum is a row reduction.
template <typename T>
__global__ __launch_bounds__(kThreads) void quant_gsum_kernel(const T* __restrict__ src, int rows,
                                                              int K, int8_t* __restrict__ q,
                                                              float* __restrict__ scale,
                                                              int* __restrict__ gsum,
                                                              int8_t* __restrict__ dbg_q,
                                                              float* __restrict__ dbg_s) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = blockIdx.x * (kThreads / kWave) + (threadIdx.x >> 6);
  if (r >= rows) return;  // uniform per wave
  const T* row = src + static_cast<size_t>(r) * K;
  const int C = K / 8;
  float amax = 0.0f;
  for (int c = lane; c < C; c += kWave) {
    float v[8];
    load8(row + c * 8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, wave_shfl_xor(amax, m));
  const float s = amax / 127.0f;
  for (int c0 = 0; c0 < C; c0 += kWave) {   // uniform trip count: all lanes reduce
    const int c = c0 + lane;
    int sum = 0;
    if (c < C) {
      float v[8];
      load8(row + c * 8, v);
      uint32_t packed[2] = {0, 0};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int code = quant_code4a8(v[i], s);
        sum += code;
        packed[i >> 2] |= (static_cast<uint32_t>(code) & 0xFFu) << (8 * (i & 3));
      }
      const uint2 pv = make_uint2(packed[0], packed[1]);
      *reinterpret_cast<uint2*>(q + static_cast<size_t>(r) * K + c * 8) = pv;
      if (dbg_q) *reinterpret_cast<uint2*>(dbg_q + static_cast<size_t>(r) * K + c * 8) = pv;
    }
    // sum over the 16 chunks of each group (16-lane rows of the wave)
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) sum += wave_shfl_xor(sum, m);
    if ((lane & 15) == 0 && c < C) gsum[static_cast<size_t>(r) * (K / 128) + c / 16] = sum;
  }
  if (lane == 0) {
    scale[r] = s;
    if (dbg_s) dbg_s[r] = s;
  }
}

// ------------------------------------------------------------- int8 GEMM ----
// KIND 0: gate/up. Wave w owns h-columns [nt*128 + 32w, +32): B subtile 0 the
//         gate rows, subtile 1 the matching up rows. Out: h float32 [R, I].
// KIND 1: down. Wave w owns W2 rows [nt*256 + 64w, +64) as two subtiles.
// K order inside a 128-k group: lane half hf takes k = 64*hf + [0, 64); MFMA
// step s (of 4) takes k = 64*hf + 16*s + [0, 16) for that half, on both
// operands (natural order: 16 consecutive codes / activation bytes).
// Per group: codes of the group (32 bytes per lane and subtile) and the raw
// fp16 scales stream through a register ring of kD groups, with this thread's
// 16-byte share of the activation tile; the activation tile is written to a
// swizzled LDS stage one step before use (two stages).
template <int KIND>
__global__ __launch_bounds__(kThreads, 2) void w4a8_mfma_kernel(
    const int8_t* __restrict__ A, const float* __restrict__ a_scale,
    const int* __restrict__ a_gsum, const uint8_t* __restrict__ W,
    const uint16_t* __restrict__ S, const int* __restrict__ offsets,
    const int* __restrict__ sorted_slot, float* __restrict__ out, int K, int N, int E, int topk,
    int NT) {
  constexpr int STAGE = kBM * 128;   // bytes of one activation stage
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[2 * STAGE];
  __shared__ int row_src[kBM];
  __shared__ float row_scale[kBM];
  __shared__ int sm_pref[kThreads / kWave];
  __shared__ int sm_out[3];
  extern __shared__ int gs_lds[];   // [kBM][G]: 8 * group code sums of the tile rows

  TileInfo ti;
  if (!find_tile<kBM>(offsets, E, NT, sm_pref, sm_out, ti)) return;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int G = K / kGroup;

  if (tid < kBM) {
    const int p = ti.p_begin + tid;
    const int pv = p < ti.p_end ? p : ti.p_begin;
    const int src = (KIND == 0) ? sorted_slot[pv] / topk : pv;
    row_src[tid] = src;
    row_scale[tid] = a_scale[src];
  }
  __syncthreads();
  for (int i = tid; i < kBM * G; i += kThreads) {
    const int m = i / G, g = i - m * G;
    gs_lds[i] = 8 * a_gsum[static_cast<size_t>(row_src[m]) * G + g];
  }

  int nrow[2];
  bool nvalid[2];
  if (KIND == 0) {
    const int n = ti.nt * 128 + wv * 32 + l32;
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
  const uint32_t rowb = static_cast<uint32_t>(K / 2);
  const __amdgpu_buffer_rsrc_t w_rsrc =
      buffer_rsrc(W + static_cast<size_t>(ti.e) * N * rowb, static_cast<uint32_t>(N) * rowb);
  const __amdgpu_buffer_rsrc_t s_rsrc =
      buffer_rsrc(S + static_cast<size_t>(ti.e) * N * G, static_cast<uint32_t>(N * G) * 2u);
  uint32_t woff[2], soff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    woff[j] = static_cast<uint32_t>(nrow[j]) * rowb + hf * 32;
    soff[j] = static_cast<uint32_t>(nrow[j] * G) * 2u;
  }
  // this thread's activation chunk: slot L = tid of a stage holds row L/8,
  // 16-byte chunk (L%8) ^ ((row/2)%8)
  const int arow = tid >> 3;
  const int8_t* asrc = A + static_cast<size_t>(row_src[arow]) * K + ((tid & 7) ^ ((arow >> 1) & 7)) * 16;
  const int adst = tid * 16;
  // LDS offsets of this lane's A operand for the 4 MFMA steps of a group
  int aoffs[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) aoffs[s] = (l32 * 8 + ((hf * 4 + s) ^ ((l32 >> 1) & 7))) * 16;

  struct Grp {
    uint4 q[2][2];
    uint32_t sc[2];
    uint4 a;
  };
  Grp ring[kD];
  auto issue = [&](int g, Grp& b) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      b.q[j][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                w_rsrc, woff[j], g * 64, 0));
      b.q[j][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                w_rsrc, woff[j] + 16, g * 64, 0));
    }
    b.a = ld16(asrc + g * kGroup);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      b.sc[j] = __builtin_amdgcn_raw_buffer_load_b16(s_rsrc, soff[j], g * 2, 0);
  };

  float acc[2][16];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;

  // 8 codes (one dword, byte b = k(2b) | k(2b+1) << 4) -> 8 int8 in k order
  auto unpack = [](uint32_t w, uint32_t& d0, uint32_t& d1) {
    const uint32_t t = w >> 4;
    d0 = __builtin_amdgcn_perm(t, w, 0x05010400u) & 0x0F0F0F0Fu;
    d1 = __builtin_amdgcn_perm(t, w, 0x07030602u) & 0x0F0F0F0Fu;
  };
  auto compute = [&](const Grp& b, int stage, int g) {
    const uint8_t* st = a_lds + stage * STAGE;
    uint4 av[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) av[s] = *reinterpret_cast<const uint4*>(st + aoffs[s]);
    __builtin_amdgcn_sched_barrier(0);
    i32x16_t accg[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) accg[j][r] = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const i32x4_t aop = __builtin_bit_cast(i32x4_t, av[s]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        // step s uses bytes [8s, 8s + 8) of the lane's 32 code bytes
        const uint32_t w0 = (&b.q[j][s >> 1].x)[(s & 1) * 2];
        const uint32_t w1 = (&b.q[j][s >> 1].x)[(s & 1) * 2 + 1];
        i32x4_t bop;
        uint32_t d0, d1, d2, d3;
        unpack(w0, d0, d1);
        unpack(w1, d2, d3);
        bop[0] = static_cast<int>(d0);
        bop[1] = static_cast<int>(d1);
        bop[2] = static_cast<int>(d2);
        bop[3] = static_cast<int>(d3);
        accg[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop, bop, accg[j], 0, 0, 0);
      }
    }
    // exact integer correction for the zero point, then the group scale
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float sc = fp16_bits_to_f32(static_cast<uint16_t>(b.sc[j]));
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = (r >> 2) * 8 + hf * 4 + (r & 3);
        acc[j][r] += sc * static_cast<float>(accg[j][r] - gs_lds[m * G + g]);
      }
    }
  };

  asm volatile("" ::"s"(out));
#pragma unroll
  for (int d = 0; d < kD - 1; ++d) issue(min(d, G - 1), ring[d]);
  *reinterpret_cast<uint4*>(a_lds + adst) = ring[0].a;
  for (int g0 = 0; g0 < G; g0 += kD) {
#pragma unroll
    for (int d = 0; d < kD; ++d) {
      const int g = g0 + d;
      __syncthreads();  // group g's stage is written; group g + 1's is free
      issue(min(g + kD - 1, G - 1), ring[(d + kD - 1) % kD]);
      if (g < G) compute(ring[d], g & 1, g);
      if (g + 1 < G)
        *reinterpret_cast<uint4*>(a_lds + ((g + 1) & 1) * STAGE + adst) = ring[(d + 1) % kD].a;
    }
  }

  // epilogue; C layout: lane holds column l32, rows 8*(r/4) + 4*hf + (r%4)
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = (r >> 2) * 8 + hf * 4 + (r & 3);
    const int p = ti.p_begin + m;
    if (p >= ti.p_end) continue;
    const float rs = row_scale[m];
    if (KIND == 0) {
      if (nvalid[0]) {
        const int n = ti.nt * 128 + wv * 32 + l32;
        out[static_cast<size_t>(p) * (N / 2) + n] = silu_mul(acc[0][r] * rs, acc[1][r] * rs);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (nvalid[j]) out[static_cast<size_t>(p) * N + nrow[j]] = acc[j][r] * rs;
    }
  }
}

template <int KIND>
hipError_t launch_w4a8_gemm(const int8_t* A, const float* a_scale, const int* a_gsum,
                            const uint8_t* W, const uint16_t* S, const int* offsets,
                            const int* sorted_slot, float* out, int K, int N, int E, int topk,
                            int T, hipStream_t s) {
  const int NT = (KIND == 0) ? (N / 2 + 127) / 128 : (N + 255) / 256;
  const long long R = static_cast<long long>(T) * topk;
  const long long act = R < E ? R : E;
  const long long mt_up = (R + kBM - 1) / kBM + act;
  long long grid = (mt_up * NT + 7) / 8 * 8;
  const size_t lds = static_cast<size_t>(kBM) * (K / kGroup) * sizeof(int);
  hipLaunchKernelGGL((w4a8_mfma_kernel<KIND>), dim3(static_cast<unsigned>(grid)), dim3(kThreads),
                     lds, s, A, a_scale, a_gsum, W, S, offsets, sorted_slot, out, K, N, E, topk,
                     NT);
  return hipGetLastError();
}

struct W4A8Ws {
  int8_t* xq;
  float* xs;
  int* xg;
  float* h;
  int8_t* hq;
  float* hs;
  int* hg;
};

W4A8Ws carve(void* ws, int T, int H, int I, int k) {
  const size_t R = static_cast<size_t>(T) * k;
  char* p = static_cast<char*>(ws);
  W4A8Ws w;
  w.xq = reinterpret_cast<int8_t*>(p);
  p += align_up(static_cast<size_t>(T) * H, 256);
  w.xs = reinterpret_cast<float*>(p);
  p += align_up(static_cast<size_t>(T) * 4, 256);
  w.xg = reinterpret_cast<int*>(p);
  p += align_up(static_cast<size_t>(T) * (H / kGroup) * 4, 256);
  w.h = reinterpret_cast<float*>(p);
  p += align_up(R * I * 4, 256);
  w.hq = reinterpret_cast<int8_t*>(p);
  p += align_up(R * I, 256);
  w.hs = reinterpret_cast<float*>(p);
  p += align_up(R * 4, 256);
  w.hg = reinterpret_cast<int*>(p);
  return w;
}

}  // namespace

size_t w4a8_workspace_bytes(int T, int H, int I, int, int k) {
  const size_t R = static_cast<size_t>(T) * k;
  return align_up(static_cast<size_t>(T) * H, 256) + align_up(static_cast<size_t>(T) * 4, 256) +
         align_up(static_cast<size_t>(T) * (H / kGroup) * 4, 256) + align_up(R * I * 4, 256) +
         align_up(R * I, 256) + align_up(R * 4, 256) + align_up(R * (I / kGroup) * 4, 256);
}

hipError_t launch_w4a8_ffn(int T, int H, int I, int E, int k, const uint16_t* x,
                           const uint8_t* w13, const uint16_t* s13, const uint8_t* w2,
                           const uint16_t* s2, const int* offsets, const int* sorted_slot,
                           float* y, const W4A8Debug& dbg, void* ws, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const W4A8Ws w = carve(ws, T, H, I, k);
  const int R = T * k;
  const int rpb = kThreads / kWave;
  quant_gsum_kernel<uint16_t><<<(T + rpb - 1) / rpb, kThreads, 0, s>>>(x, T, H, w.xq, w.xs, w.xg,
                                                                       dbg.xq, dbg.xs);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  err = launch_w4a8_gemm<0>(w.xq, w.xs, w.xg, w13, s13, offsets, sorted_slot, w.h, H, 2 * I, E, k,
                            T, s);
  if (err != hipSuccess) return err;
  quant_gsum_kernel<float><<<(R + rpb - 1) / rpb, kThreads, 0, s>>>(w.h, R, I, w.hq, w.hs, w.hg,
                                                                    dbg.hq, dbg.hs);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_w4a8_gemm<1>(w.hq, w.hs, w.hg, w2, s2, offsets, sorted_slot, y, I, H, E, k, T, s);
}

}  // namespace moe
