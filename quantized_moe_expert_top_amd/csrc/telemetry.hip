// Expert-load telemetry: per-expert routed-row counts accumulated over calls,
// and each layer's experts ranked by load.
//
// "Performance and verification", section "Why it is fast": the engines count
// their own routing as they run and move the experts used most. The counts
// are the lengths of the expert blocks of the permutation (expert_offsets);
// the ranking is by descending load, ties to the lower expert index.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// counts[l, e] += offsets_l[e + 1] - offsets_l[e]; one thread per (l, e).
// Calls on one stream are ordered, so the read-modify-write needs no atomic.
__global__ __launch_bounds__(kThreads) void expert_counts_kernel(
    const int* __restrict__ offsets, long long stride, int E, unsigned long long* __restrict__ counts) {
  const int e = blockIdx.x * kThreads + threadIdx.x;
  const int l = blockIdx.y;
  if (e >= E) return;
  const int* o = offsets + static_cast<size_t>(l) * stride;
  const int rows = o[e + 1] - o[e];
  unsigned long long* c = counts + static_cast<size_t>(l) * E + e;
  *c += static_cast<unsigned long long>(rows);
}

// One block per layer, one thread per expert (E <= 1024): an expert's place
// in the ranking is the number of experts ahead of it (a larger load, or an
// equal load and a lower index); places below n are written out.
__global__ __launch_bounds__(1024) void hot_rank_kernel(const unsigned long long* __restrict__ counts,
                                                        int E, int n, int* __restrict__ hot) {
  __shared__ unsigned long long c[1024];
  const int t = threadIdx.x, l = blockIdx.x;
  const unsigned long long* cl = counts + static_cast<size_t>(l) * E;
  if (t < E) c[t] = cl[t];
  __syncthreads();
  if (t >= E) return;
  const unsigned long long mine = c[t];
  int place = 0;
  for (int j = 0; j < E; ++j) {
    const unsigned long long cj = c[j];
    place += (cj > mine) || (cj == mine && j < t);
  }
  if (place < n) hot[static_cast<size_t>(l) * n + place] = t;
}

}  // namespace

hipError_t launch_expert_counts(const int* offsets, long long stride, int L, int E,
                                unsigned long long* counts, hipStream_t s) {
  if (L == 0) return hipSuccess;
  hipLaunchKernelGGL(expert_counts_kernel, dim3((E + kThreads - 1) / kThreads, L), dim3(kThreads),
                     0, s, offsets, stride, E, counts);
  return hipGetLastError();
}

hipError_t launch_hot_rank(const unsigned long long* counts, int L, int E, int n, int* hot,
                           hipStream_t s) {
  if (L == 0 || n == 0) return hipSuccess;
  const int threads = (E + kWave - 1) / kWave * kWave;
  hipLaunchKernelGGL(hot_rank_kernel, dim3(L), dim3(threads), 0, s, counts, E, n, hot);
  return hipGetLastError();
}

}  // namespace moe
