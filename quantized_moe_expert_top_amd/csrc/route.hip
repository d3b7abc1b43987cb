// Top-k routing: one wavefront per token.
//
// Each lane holds E/64 router logits as 64-bit keys
//   key = orderable(logit) << 32 | (0xFFFFFFFF - expert)
// so the unsigned maximum is the largest logit with the lowest expert index on
// ties (+0.0 and -0.0 are made equal first). k rounds of a wave-wide max pick
// the experts in descending order; the owner lane clears the winner's key.
// Router ids are integer outputs and must be exact ("Performance and
// verification", section "How it is verified"); the weights are a float32
// softmax over the k selected logits.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

__device__ __forceinline__ uint64_t route_key(float l, int e) {
  uint32_t b = __float_as_uint(l);
  if (b == 0x80000000u) b = 0u;  // -0.0 ties +0.0
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (static_cast<uint64_t>(ord) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(e));
}

template <int S>  // key slots per lane: E <= 64 * S
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int* __restrict__ ids,
                                                         float* __restrict__ w) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  const float* row = logits + static_cast<size_t>(t) * E;

  uint64_t key[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int e = lane + kWave * s;
    key[s] = (e < E) ? route_key(row[e], e) : 0ull;  // valid keys are > 0
  }

  int my_e = 0;
  float my_l = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int s = 1; s < S; ++s) best = key[s] > best ? key[s] : best;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const uint64_t o = wave_shfl_xor(best, m);
      best = o > best ? o : best;
    }
#pragma unroll
    for (int s = 0; s < S; ++s)
      if (key[s] == best) key[s] = 0ull;
    const int e = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best));
    if (lane == j) {
      my_e = e;
      my_l = row[e];
    }
  }

  // softmax over the k picks; pick 0 holds the maximum
  const float lmax = __shfl(my_l, 0, kWave);
  const float z = (lane < k) ? expf(my_l - lmax) : 0.0f;
  float sum = z;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) sum += wave_shfl_xor(sum, m);
  if (lane < k) {
    ids[static_cast<size_t>(t) * k + lane] = my_e;
    w[static_cast<size_t>(t) * k + lane] = z / sum;
  }
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int* ids, float* w,
                             hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((T + 3) / 4), block(256);
  if (E <= 64)
    route_topk_kernel<1><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else if (E <= 128)
    route_topk_kernel<2><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else if (E <= 256)
    route_topk_kernel<4><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else if (E <= 512)
    route_topk_kernel<8><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else
    route_topk_kernel<16><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace moe
