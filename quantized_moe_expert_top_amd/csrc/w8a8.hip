// Grouped SwiGLU expert FFN on int8 x int8 -> int32 MFMA (W8A8).
//
// "Performance and verification", section "Why it is fast": routed experts of
// a prompt run as grouped int8 tensor-core GEMMs. Here:
//   1. act_quant: per token row, s = absmax/127 (IEEE float32 division), codes
//      rint(x/s) clamped to [-127, 127] (round half to even).
//   2. gate/up: v_mfma_i32_32x32x32_i8 over (expert, 128-row, 64-column) tiles;
//      the epilogue dequantizes (acc * xs[t] * s13[e,n]) and applies SwiGLU in
//      float32, writing h (float32) in grouped order.
//   3. h_quant: the same per-row rule on h (one row per routed slot). h stays
//      float32 until here so the code decisions match a float32 reference.
//   4. down: int8 MFMA over (expert, 128-row, 128-column) tiles; y = acc *
//      hs[p] * s2[e,n], stored float32.
// The int32 accumulators are exact, so they are reproducible bit for bit.
#include "common.h"
#include "launch.h"
#include "tiles.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kBM = 128;        // rows per tile
constexpr int kBK = 64;         // K per pipeline step (two MFMA k-steps of 32)
constexpr int kLd = kBK + 16;   // LDS row stride in bytes (bank spread)

// --------------------------------------------------------- quantization ----
__device__ __forceinline__ int8_t quant_code(float v, float s) {
  if (s == 0.0f) return 0;
  float q = rintf(v / s);
  q = fminf(fmaxf(q, -127.0f), 127.0f);
  return static_cast<int8_t>(static_cast<int>(q));
}

// One wave per token row of x (bf16 [T, H]); H % 8 == 0.
__global__ __launch_bounds__(kThreads) void act_quant_kernel(const uint16_t* __restrict__ x,
                                                             int T, int H,
                                                             int8_t* __restrict__ xq,
                                                             float* __restrict__ xs,
                                                             int8_t* __restrict__ dbg_xq,
                                                             float* __restrict__ dbg_xs) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (kThreads / kWave) + (threadIdx.x >> 6);
  if (t >= T) return;
  const uint16_t* row = x + static_cast<size_t>(t) * H;
  float amax = 0.0f;
  for (int c = lane * 8; c < H; c += kWave * 8) {
    const uint4 v = ld16(row + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      amax = fmaxf(amax, fmaxf(fabsf(bf16lo(w[i])), fabsf(bf16hi(w[i]))));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, wave_shfl_xor(amax, m));
  const float s = amax / 127.0f;
  for (int c = lane * 8; c < H; c += kWave * 8) {
    const uint4 v = ld16(row + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t packed[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = static_cast<uint8_t>(quant_code(bf16lo(w[i]), s));
      const uint32_t hi = static_cast<uint8_t>(quant_code(bf16hi(w[i]), s));
      packed[i >> 1] |= (lo | (hi << 8)) << (16 * (i & 1));
    }
    const uint2 pv = make_uint2(packed[0], packed[1]);
    *reinterpret_cast<uint2*>(xq + static_cast<size_t>(t) * H + c) = pv;
    if (dbg_xq) *reinterpret_cast<uint2*>(dbg_xq + static_cast<size_t>(t) * H + c) = pv;
  }
  if (lane == 0) {
    xs[t] = s;
    if (dbg_xs) dbg_xs[t] = s;
  }
}

// One wave per routed row of h (float32 [R, I]); I % 4 == 0.
__global__ __launch_bounds__(kThreads) void h_quant_kernel(const float* __restrict__ h, int R,
                                                           int I, int8_t* __restrict__ hq,
                                                           float* __restrict__ hs,
                                                           int8_t* __restrict__ dbg_hq,
                                                           float* __restrict__ dbg_hs) {
  const int lane = threadIdx.x & (kWave - 1);
  const int p = blockIdx.x * (kThreads / kWave) + (threadIdx.x >> 6);
  if (p >= R) return;
  const float* row = h + static_cast<size_t>(p) * I;
  float amax = 0.0f;
  for (int c = lane * 4; c < I; c += kWave * 4) {
    const float4 v = *reinterpret_cast<const float4*>(row + c);
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, wave_shfl_xor(amax, m));
  const float s = amax / 127.0f;
  for (int c = lane * 4; c < I; c += kWave * 4) {
    const float4 v = *reinterpret_cast<const float4*>(row + c);
    const uint32_t q = static_cast<uint8_t>(quant_code(v.x, s)) |
                       (static_cast<uint32_t>(static_cast<uint8_t>(quant_code(v.y, s))) << 8) |
                       (static_cast<uint32_t>(static_cast<uint8_t>(quant_code(v.z, s))) << 16) |
                       (static_cast<uint32_t>(static_cast<uint8_t>(quant_code(v.w, s))) << 24);
    *reinterpret_cast<uint32_t*>(hq + static_cast<size_t>(p) * I + c) = q;
    if (dbg_hq) *reinterpret_cast<uint32_t*>(dbg_hq + static_cast<size_t>(p) * I + c) = q;
  }
  if (lane == 0) {
    hs[p] = s;
    if (dbg_hs) dbg_hs[p] = s;
  }
}

// ------------------------------------------------------------- int8 GEMM ----
// KIND 0: gate/up. Tile = 128 rows x 64 h-columns; wave (wm, wn) owns rows
//         [64wm, +64) and h-columns [32wn, +32): B subtile 0 = gate rows,
//         subtile 1 = the matching up rows. Out: h float32 [R, I].
// KIND 1: down. Tile = 128 rows x 128 W2 rows; wave (wm, wn) owns rows
//         [64wm, +64) and W2 rows [64wn, +64) as two subtiles. Out: y float32.
// LDS holds the A tile (128 x 64 int8) and the B tile (128 W rows x 64 int8)
// per pipeline step, double-buffered. Operand k order inside one MFMA step:
// lane half hf = lane/32 takes k = 32*ks + 16*hf + [0, 16).
template <int KIND>
__global__ __launch_bounds__(kThreads) void w8a8_mfma_kernel(
    const int8_t* __restrict__ A, const float* __restrict__ a_scale,
    const int8_t* __restrict__ W, const float* __restrict__ w_scale,
    const int* __restrict__ offsets, const int* __restrict__ sorted_slot, int K, int N, int E,
    int topk, int NT, float* __restrict__ h_out, float* __restrict__ y_out,
    int32_t* __restrict__ dbg_acc) {
  __shared__ __attribute__((aligned(16))) int8_t a_lds[2][kBM * kLd];
  __shared__ __attribute__((aligned(16))) int8_t b_lds[2][kBM * kLd];
  __shared__ int row_src[kBM];
  __shared__ int sm_pref[kThreads / kWave];
  __shared__ int sm_out[3];

  TileInfo ti;
  if (!find_tile<kBM>(offsets, E, NT, sm_pref, sm_out, ti)) return;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int wm = wv >> 1, wn = wv & 1;
  const int I = N / 2;  // KIND 0 only

  // source row of each A tile row (token for gate/up, grouped row for down)
  if (tid < kBM) {
    const int p = ti.p_begin + tid;
    row_src[tid] = (p < ti.p_end) ? ((KIND == 0) ? sorted_slot[p] / topk : p) : -1;
  }
  // W row held at B tile row j (0..127)
  auto b_row = [&](int j) -> int {
    if (KIND == 0) {
      const int half = j >> 6, c = ti.nt * 64 + (j & 63);
      const int cc = c < I ? c : I - 1;
      return half * I + cc;
    } else {
      const int r = ti.nt * 128 + j;
      return r < N ? r : N - 1;
    }
  };
  __syncthreads();

  // each thread moves 2 A chunks and 2 B chunks of 16 bytes per step
  const int8_t* asrc[2];
  const int8_t* bsrc[2];
  int aoff[2];
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    const int q = tid + kThreads * v;       // 0..511
    const int r = q >> 2, ch = q & 3;       // row 0..127, 16-byte chunk 0..3
    const int src = row_src[r];
    asrc[v] = (src >= 0) ? A + static_cast<size_t>(src) * K + ch * 16 : nullptr;
    bsrc[v] = W + (static_cast<size_t>(ti.e) * N + b_row(r)) * K + ch * 16;
    aoff[v] = r * kLd + ch * 16;
  }

  i32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  uint4 ar[2], br[2];
  auto gload = [&](int step) {
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      ar[v] = asrc[v] ? ld16(asrc[v] + step * kBK) : make_uint4(0, 0, 0, 0);
      br[v] = ld16(bsrc[v] + step * kBK);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      *reinterpret_cast<uint4*>(&a_lds[buf][aoff[v]]) = ar[v];
      *reinterpret_cast<uint4*>(&b_lds[buf][aoff[v]]) = br[v];
    }
  };

  const int steps = K / kBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int st = 0; st < steps; ++st) {
    const int buf = st & 1;
    const bool more = st + 1 < steps;
    if (more) gload(st + 1);
#pragma unroll
    for (int ks = 0; ks < kBK / 32; ++ks) {
      i32x4_t bop[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int brow = (KIND == 0) ? (j * 64 + wn * 32 + l32) : (wn * 64 + j * 32 + l32);
        bop[j] = *reinterpret_cast<const i32x4_t*>(&b_lds[buf][brow * kLd + ks * 32 + hf * 16]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int arow = wm * 64 + i * 32 + l32;
        const i32x4_t aop =
            *reinterpret_cast<const i32x4_t*>(&a_lds[buf][arow * kLd + ks * 32 + hf * 16]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop, bop[j], acc[i][j], 0, 0, 0);
      }
    }
    if (more) sstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue; C layout: lane holds column l32, rows 8*(r/4) + 4*hf + (r%4)
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = wm * 64 + i * 32 + (r >> 2) * 8 + hf * 4 + (r & 3);
      const int p = ti.p_begin + m;
      if (p >= ti.p_end) continue;
      if (KIND == 0) {
        const int n = ti.nt * 64 + wn * 32 + l32;
        if (n >= I) continue;
        const int ag = acc[i][0][r], au = acc[i][1][r];
        if (dbg_acc) {
          dbg_acc[static_cast<size_t>(p) * N + n] = ag;
          dbg_acc[static_cast<size_t>(p) * N + I + n] = au;
        }
        const float xs = a_scale[row_src[m]];
        const float g = static_cast<float>(ag) * xs * w_scale[static_cast<size_t>(ti.e) * N + n];
        const float u = static_cast<float>(au) * xs * w_scale[static_cast<size_t>(ti.e) * N + I + n];
        h_out[static_cast<size_t>(p) * I + n] = silu_mul(g, u);
      } else {
        const float hsv = a_scale[p];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = ti.nt * 128 + wn * 64 + j * 32 + l32;
          if (n >= N) continue;
          const int a = acc[i][j][r];
          if (dbg_acc) dbg_acc[static_cast<size_t>(p) * N + n] = a;
          y_out[static_cast<size_t>(p) * N + n] =
              static_cast<float>(a) * hsv * w_scale[static_cast<size_t>(ti.e) * N + n];
        }
      }
    }
  }
}

template <int KIND>
hipError_t launch_w8a8_gemm(const int8_t* A, const float* a_scale, const int8_t* W,
                            const float* w_scale, const int* offsets, const int* sorted_slot,
                            int K, int N, int E, int topk, int T, float* h_out, float* y_out,
                            int32_t* dbg_acc, hipStream_t s) {
  const int NT = (KIND == 0) ? (N / 2 + 63) / 64 : (N + 127) / 128;
  const long long R = static_cast<long long>(T) * topk;
  const long long act = R < E ? R : E;
  const long long mt_up = (R + kBM - 1) / kBM + act;
  long long grid = (mt_up * NT + 7) / 8 * 8;
  hipLaunchKernelGGL((w8a8_mfma_kernel<KIND>), dim3(static_cast<unsigned>(grid)), dim3(kThreads),
                     0, s, A, a_scale, W, w_scale, offsets, sorted_slot, K, N, E, topk, NT, h_out,
                     y_out, dbg_acc);
  return hipGetLastError();
}

struct W8A8Ws {
  int8_t* xq;
  float* xs;
  float* h;
  int8_t* hq;
  float* hs;
};

W8A8Ws carve(void* ws, int T, int H, int I, int k) {
  const size_t R = static_cast<size_t>(T) * k;
  char* p = static_cast<char*>(ws);
  W8A8Ws w;
  w.xq = reinterpret_cast<int8_t*>(p);
  p += align_up(static_cast<size_t>(T) * H, 256);
  w.xs = reinterpret_cast<float*>(p);
  p += align_up(static_cast<size_t>(T) * 4, 256);
  w.h = reinterpret_cast<float*>(p);
  p += align_up(R * I * 4, 256);
  w.hq = reinterpret_cast<int8_t*>(p);
  p += align_up(R * I, 256);
  w.hs = reinterpret_cast<float*>(p);
  return w;
}

}  // namespace

size_t w8a8_workspace_bytes(int T, int H, int I, int, int k) {
  const size_t R = static_cast<size_t>(T) * k;
  return align_up(static_cast<size_t>(T) * H, 256) + align_up(static_cast<size_t>(T) * 4, 256) +
         align_up(R * I * 4, 256) + align_up(R * I, 256) + align_up(R * 4, 256);
}

hipError_t launch_w8a8_ffn(int T, int H, int I, int E, int k, const uint16_t* x,
                           const int8_t* w13, const float* s13, const int8_t* w2,
                           const float* s2, const int* offsets, const int* sorted_slot,
                           const int*, const int*, float* y, const W8A8Debug& dbg, void* ws,
                           hipStream_t s) {
  if (T == 0) return hipSuccess;
  const W8A8Ws w = carve(ws, T, H, I, k);
  const int R = T * k;
  const int rows_per_block = kThreads / kWave;
  act_quant_kernel<<<(T + rows_per_block - 1) / rows_per_block, kThreads, 0, s>>>(
      x, T, H, w.xq, w.xs, dbg.xq, dbg.xs);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  err = launch_w8a8_gemm<0>(w.xq, w.xs, w13, s13, offsets, sorted_slot, H, 2 * I, E, k, T, w.h,
                            nullptr, dbg.acc13, s);
  if (err != hipSuccess) return err;
  h_quant_kernel<<<(R + rows_per_block - 1) / rows_per_block, kThreads, 0, s>>>(
      w.h, R, I, w.hq, w.hs, dbg.hq, dbg.hs);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_w8a8_gemm<1>(w.hq, w.hs, w2, s2, offsets, sorted_slot, I, H, E, k, T, nullptr, y,
                             dbg.acc2, s);
}

}  // namespace moe
