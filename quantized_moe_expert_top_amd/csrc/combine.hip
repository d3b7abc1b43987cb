// Weighted combine of each token's k expert outputs, in a fixed order.
//
// out[t, :] = sum_j w[t, j] * y[slot_pos[t*k + j], :], accumulated in float32
// in increasing j. No float atomics: each output element is owned by one
// thread, so the result is bitwise reproducible.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

// Each thread owns 8 consecutive floats of one token's row. The picks are
// taken in full batches of kJB: a batch's slot positions and weights are
// loaded together, then all of its y reads are issued before the first is
// used, so the batch costs one round trip to memory for the positions and one
// for the rows (loading and adding one pick at a time waits k times). Picks
// left over past the last full batch go one at a time. The adds run in
// increasing j either way.
constexpr int kJB = 8;

__device__ __forceinline__ void add_pick(float (&acc)[8], float wj, const float4& a,
                                         const float4& b) {
  acc[0] += wj * a.x;
  acc[1] += wj * a.y;
  acc[2] += wj * a.z;
  acc[3] += wj * a.w;
  acc[4] += wj * b.x;
  acc[5] += wj * b.y;
  acc[6] += wj * b.z;
  acc[7] += wj * b.w;
}

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int* __restrict__ slot_pos,
                                                      const float* __restrict__ w, int T, int H,
                                                      int k, float* __restrict__ out) {
  const int chunks = H / 8;
  const long long idx = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<long long>(T) * chunks) return;
  const int t = static_cast<int>(idx / chunks);
  const int c = static_cast<int>(idx % chunks);
  const int* sp = slot_pos + static_cast<size_t>(t) * k;
  const float* wt = w + static_cast<size_t>(t) * k;
  const float* yc = y + c * 8;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int j0 = 0;
  for (; j0 + kJB <= k; j0 += kJB) {
    int p[kJB];
    float wj[kJB];
#pragma unroll
    for (int u = 0; u < kJB; ++u) {
      p[u] = sp[j0 + u];
      wj[u] = wt[j0 + u];
    }
    float4 a[kJB], b[kJB];
#pragma unroll
    for (int u = 0; u < kJB; ++u) {
      const float4* src = reinterpret_cast<const float4*>(yc + static_cast<size_t>(p[u]) * H);
      a[u] = src[0];
      b[u] = src[1];
    }
    __builtin_amdgcn_sched_barrier(0);   // all of the batch's reads go out first
#pragma unroll
    for (int u = 0; u < kJB; ++u) add_pick(acc, wj[u], a[u], b[u]);
  }
  for (int j = j0; j < k; ++j) {
    const float4* src = reinterpret_cast<const float4*>(yc + static_cast<size_t>(sp[j]) * H);
    add_pick(acc, wt[j], src[0], src[1]);
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
