// Streaming-read ceiling probe for one MI355X: back-to-back launches of a
// plain 16-byte-load read kernel over slabs rotated through a 1 GiB buffer
// (so consecutive launches do not reuse the MALL), timed with HIP events;
// plus the back-to-back cost of an empty kernel. With the argument "copy" it
// runs a plain copy of known size instead, the reference dispatch for
// calibrating the FETCH_SIZE and WRITE_SIZE counters.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <vector>
#define CK(x) do { hipError_t e = (x); if (e != hipSuccess) { printf("err %s line %d\n", hipGetErrorString(e), __LINE__); return 1; } } while (0)
// each thread reads PER x 16B at stride blockDim*16 within its block's slab
template <int PER>
__global__ __launch_bounds__(256) void rd(const uint4* __restrict__ p, size_t slab_u4, unsigned* out) {
  const uint4* b = p + blockIdx.x * slab_u4;
  unsigned acc = 0;
  uint4 v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) v[i] = b[threadIdx.x + i * 256];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  if (acc == 0x12345678u) out[blockIdx.x] = acc;
}
__global__ void empty_k(unsigned* out) { if (threadIdx.x == 12345) out[0] = 1; }
// plain copy: each thread moves 8 x 16 B (one known-size read and write stream)
__global__ __launch_bounds__(256) void cp(const uint4* __restrict__ src, uint4* __restrict__ dst) {
  const size_t base = static_cast<size_t>(blockIdx.x) * 2048 + threadIdx.x;
  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = src[base + i * 256];
#pragma unroll
  for (int i = 0; i < 8; ++i) dst[base + i * 256] = v[i];
}
// "copy" mode: three launches of cp over 256 MiB (src) -> 256 MiB (dst); the
// counter calibration divides what FETCH_SIZE / WRITE_SIZE report for these
// dispatches by the 262144 KiB each of them moves.
int copy_mode() {
  const size_t bytes = size_t(256) << 20;
  uint4 *src, *dst;
  CK(hipMalloc(&src, bytes)); CK(hipMalloc(&dst, bytes));
  CK(hipMemset(src, 1, bytes)); CK(hipMemset(dst, 0, bytes));
  CK(hipDeviceSynchronize());
  const int blocks = static_cast<int>(bytes / (2048 * 16));
  for (int i = 0; i < 3; ++i) cp<<<blocks, 256>>>(src, dst);
  CK(hipDeviceSynchronize());
  printf("copy: 3 dispatches, each reads and writes %zu KiB\n", bytes >> 10);
  return 0;
}
int main(int argc, char** argv) {
  if (argc > 1 && argv[1][0] == 'c') return copy_mode();
  size_t maxbytes = size_t(1) << 30;
  uint4* buf; unsigned* out;
  CK(hipMalloc(&buf, maxbytes)); CK(hipMalloc(&out, 1 << 20));
  CK(hipMemset(buf, 1, maxbytes));
  hipEvent_t a, b; CK(hipEventCreate(&a)); CK(hipEventCreate(&b));
  const int iters = 200;
  // empty kernel
  for (int w = 0; w < 10; ++w) empty_k<<<1, 64>>>(out);
  CK(hipEventRecord(a)); for (int i = 0; i < iters; ++i) empty_k<<<1, 64>>>(out); CK(hipEventRecord(b)); CK(hipEventSynchronize(b));
  float ms; CK(hipEventElapsedTime(&ms, a, b)); printf("empty kernel back-to-back: %.2f us each\n", ms * 1000 / iters);
  // reads: blocks x 256 threads x PER x 16B; rotate base so consecutive launches don't hit MALL
  int blocks_list[] = {256, 768, 1536, 3072, 6144, 12288};
  for (int bl : blocks_list) {
    const int PER = 8;
    size_t bytes = size_t(bl) * 256 * PER * 16;
    size_t slab = 256 * PER;
    int nrot = (int)(maxbytes / bytes); if (nrot > 16) nrot = 16;
    for (int w = 0; w < 5; ++w) rd<8><<<bl, 256>>>(buf, slab, out);
    CK(hipEventRecord(a));
    for (int i = 0; i < iters; ++i) rd<8><<<bl, 256>>>(buf + (size_t)(i % nrot) * bytes / 16, slab, out);
    CK(hipEventRecord(b)); CK(hipEventSynchronize(b));
    CK(hipEventElapsedTime(&ms, a, b));
    double us = ms * 1000 / iters;
    printf("read %8.2f MB: %7.2f us/kernel -> %7.1f GB/s (rotation %d)\n", bytes / 1e6, us, bytes / us / 1e3, nrot);
  }
  return 0;
}
