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

template <int S>  // key slots per lane: E <= 64 * S
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int* __restrict__ ids,
                                                         float* __restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  wave_topk<S>(logits + static_cast<size_t>(t) * E, E, k, ids + static_cast<size_t>(t) * k,
               w + static_cast<size_t>(t) * k);
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
