// Router projection ahead of the top-k: logits[t, e] = x[t, :] . w_r[e, :].
//
// Many tokens: one v_mfma_f32_32x32x16_bf16 tile per block: 32 tokens x 32 experts. The
// four waves of a block split H into contiguous quarters; their partial tiles
// are added in LDS in wave order, so the sum order is fixed (deterministic).
// bf16 x bf16 products are exact in float32; accumulation is float32.
// Operands come straight from global memory (the router rows are small and
// stay in L2): lane (l32, hf) of a 16-k step holds 8 consecutive k of token /
// expert row l32, k = 16s + 8hf + [0, 8); four steps are requested ahead.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kAhead = 4;   // 16-k steps in flight per wave

__global__ __launch_bounds__(kThreads) void router_logits_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int H, int E,
    float* __restrict__ logits) {
  __shared__ float part[3][16][kWave];   // waves 1..3: their 16 accumulators per lane
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int t0 = blockIdx.x * 32, e0 = blockIdx.y * 32;
  // rows past the batch / the expert count read the last valid row; their
  // results are not stored
  const int t = min(t0 + l32, T - 1), e = min(e0 + l32, E - 1);
  const int kq = H / 4, steps = kq / 16;
  const uint16_t* xa = x + static_cast<size_t>(t) * H + wv * kq + hf * 8;
  const uint16_t* wb = wr + static_cast<size_t>(e) * H + wv * kq + hf * 8;

  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  uint4 ra[kAhead], rb[kAhead];
#pragma unroll
  for (int d = 0; d < kAhead; ++d) {
    const int s = min(d, steps - 1);
    ra[d] = ld16(xa + s * 16);
    rb[d] = ld16(wb + s * 16);
  }
  for (int s0 = 0; s0 < steps; s0 += kAhead) {
#pragma unroll
    for (int d = 0; d < kAhead; ++d) {
      const int s = s0 + d;
      if (s < steps) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, ra[d]),
                                                      __builtin_bit_cast(bf16x8_t, rb[d]), acc,
                                                      0, 0, 0);
        const int sn = min(s + kAhead, steps - 1);
        ra[d] = ld16(xa + sn * 16);
        rb[d] = ld16(wb + sn * 16);
      }
    }
  }
  if (wv > 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) part[wv - 1][r][lane] = acc[r];
  }
  __syncthreads();
  if (wv == 0) {
    // C layout: lane holds column l32 (expert), rows 8*(r/4) + 4*hf + (r%4)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v = acc[r];
      v += part[0][r][lane];
      v += part[1][r][lane];
      v += part[2][r][lane];
      const int tt = t0 + (r >> 2) * 8 + hf * 4 + (r & 3), ee = e0 + l32;
      if (tt < T && ee < E) logits[static_cast<size_t>(tt) * E + ee] = v;
    }
  }
}

// Few tokens (T <= kGemvT): one wave per expert row, so E waves share the
// router rows instead of E/32 tiles. Lane l takes the 16-byte chunks l,
// l + 64, ... of the row and of each token row, accumulates v_dot2 products
// per token, and the wave sum (fixed DPP order) gives the logit.
constexpr int kGemvT = 8;

template <int NT>
__global__ __launch_bounds__(kThreads) void router_gemv_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int H, int E,
    float* __restrict__ logits) {
  const int lane = threadIdx.x & (kWave - 1);
  const int e_raw = blockIdx.x * (kThreads / kWave) + (threadIdx.x >> 6);
  const int e = min(e_raw, E - 1);   // past E: a valid row, not stored
  const int C = H / 8;               // 16-byte chunks per row
  const uint16_t* w = wr + static_cast<size_t>(e) * H;
  float acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = 0.0f;
#pragma unroll 4
  for (int c = lane; c < C; c += kWave) {
    const uint4 wv = ld16(w + c * 8);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t < T) {
        const uint4 xv = ld16(x + static_cast<size_t>(t) * H + c * 8);
        acc[t] = dot2_bf16(wv.x, xv.x, acc[t]);
        acc[t] = dot2_bf16(wv.y, xv.y, acc[t]);
        acc[t] = dot2_bf16(wv.z, xv.z, acc[t]);
        acc[t] = dot2_bf16(wv.w, xv.w, acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (t < T) {
      const float v = wave_sum_f32(acc[t]);
      if (lane == 0 && e_raw < E) logits[static_cast<size_t>(t) * E + e] = v;
    }
  }
}

}  // namespace

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr, int T, int H, int E,
                                float* logits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (T <= kGemvT) {
    const int blocks = (E + kThreads / kWave - 1) / (kThreads / kWave);
    if (T <= 2)
      router_gemv_kernel<2><<<blocks, kThreads, 0, s>>>(x, wr, T, H, E, logits);
    else if (T <= 4)
      router_gemv_kernel<4><<<blocks, kThreads, 0, s>>>(x, wr, T, H, E, logits);
    else
      router_gemv_kernel<8><<<blocks, kThreads, 0, s>>>(x, wr, T, H, E, logits);
    return hipGetLastError();
  }
  const dim3 grid((T + 31) / 32, (E + 31) / 32), block(kThreads);
  router_logits_kernel<<<grid, block, 0, s>>>(x, wr, T, H, E, logits);
  return hipGetLastError();
}

}  // namespace moe
