// Weighted combine of each token's k expert outputs, in a fixed order.
//
// out[t, :] = sum_j w[t, j] * y[slot_pos[t*k + j], :], accumulated in float32
// in increasing j. No float atomics: each output element is owned by one
// thread, so the result is bitwise reproducible.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int* __restrict__ slot_pos,
                                                      const float* __restrict__ w, int T, int H,
                                                      int k, float* __restrict__ out) {
  const int chunks = H / 8;
  const long long idx = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<long long>(T) * chunks) return;
  const int t = static_cast<int>(idx / chunks);
  const int c = static_cast<int>(idx % chunks);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int j = 0; j < k; ++j) {
    const float wj = w[static_cast<size_t>(t) * k + j];
    const int p = slot_pos[static_cast<size_t>(t) * k + j];
    const float4* src = reinterpret_cast<const float4*>(y + static_cast<size_t>(p) * H + c * 8);
    const float4 a = src[0], b = src[1];
    acc[0] += wj * a.x;
    acc[1] += wj * a.y;
    acc[2] += wj * a.z;
    acc[3] += wj * a.w;
    acc[4] += wj * b.x;
    acc[5] += wj * b.y;
    acc[6] += wj * b.z;
    acc[7] += wj * b.w;
  }
  float4* o = reinterpret_cast<float4*>(out + static_cast<size_t>(t) * H + c * 8);
  o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

}  // namespace

hipError_t launch_combine(const float* y, const int* slot_pos, const float* w, int T, int H,
                          int k, float* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const long long n = static_cast<long long>(T) * (H / 8);
  const int blocks = static_cast<int>((n + 255) / 256);
  combine_kernel<<<blocks, 256, 0, s>>>(y, slot_pos, w, T, H, k, out);
  return hipGetLastError();
}

}  // namespace moe
