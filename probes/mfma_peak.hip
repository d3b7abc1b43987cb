// MFMA-only ceiling probe for one MI355X: every wave runs four independent
// chains of dense MFMAs on register operands (no memory traffic inside the
// loop; one store per thread at the end keeps the work live), launched as four
// 256-thread blocks per CU and timed with HIP events. Reports the achieved
// dense rate of v_mfma_f32_32x32x16_bf16 (TFLOP/s) and v_mfma_i32_32x32x32_i8
// (TOP/s), with the device's compute-unit count and peak clock.
#include <hip/hip_runtime.h>
#include <cstdio>
#define CK(x) do { hipError_t e = (x); if (e != hipSuccess) { printf("err %s line %d\n", hipGetErrorString(e), __LINE__); return 1; } } while (0)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));

constexpr int kChains = 4;
constexpr int kIters = 4096;

__global__ __launch_bounds__(256) void mfma_bf16(float* out, float seed) {
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(seed * (threadIdx.x + i));
    b[i] = static_cast<__bf16>(seed * (i + 1));
  }
  f32x16_t acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void mfma_i8(int* out, int seed) {
  i32x4_t a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = seed * static_cast<int>(threadIdx.x + i);
    b[i] = seed + i;
  }
  i32x16_t acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0;
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j)
      acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[j], 0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

int main() {
  hipDeviceProp_t prop;
  CK(hipGetDeviceProperties(&prop, 0));
  const int cus = prop.multiProcessorCount;
  printf("device %s: %d compute units, peak clock %.0f MHz\n", prop.gcnArchName, cus,
         prop.clockRate / 1000.0);
  const int blocks = 4 * cus;
  void* out;
  CK(hipMalloc(&out, static_cast<size_t>(blocks) * 256 * sizeof(float)));
  hipEvent_t t0, t1;
  CK(hipEventCreate(&t0));
  CK(hipEventCreate(&t1));
  const int reps = 5;
  const double waves = blocks * 4.0;
  // bf16: 32 x 32 x 16 x 2 flop per instruction
  for (int w = 0; w < 2; ++w) mfma_bf16<<<blocks, 256>>>(static_cast<float*>(out), 1e-3f);
  CK(hipEventRecord(t0));
  for (int r = 0; r < reps; ++r) mfma_bf16<<<blocks, 256>>>(static_cast<float*>(out), 1e-3f);
  CK(hipEventRecord(t1));
  CK(hipEventSynchronize(t1));
  float ms;
  CK(hipEventElapsedTime(&ms, t0, t1));
  double ops = waves * kIters * kChains * 32.0 * 32 * 16 * 2 * reps;
  printf("v_mfma_f32_32x32x16_bf16: %.1f TFLOP/s dense (%.3f ms per launch)\n",
         ops / (ms * 1e-3) / 1e12, ms / reps);
  // int8: 32 x 32 x 32 x 2 op per instruction
  for (int w = 0; w < 2; ++w) mfma_i8<<<blocks, 256>>>(static_cast<int*>(out), 3);
  CK(hipEventRecord(t0));
  for (int r = 0; r < reps; ++r) mfma_i8<<<blocks, 256>>>(static_cast<int*>(out), 3);
  CK(hipEventRecord(t1));
  CK(hipEventSynchronize(t1));
  CK(hipEventElapsedTime(&ms, t0, t1));
  ops = waves * kIters * kChains * 32.0 * 32 * 32 * 2 * reps;
  printf("v_mfma_i32_32x32x32_i8: %.1f TOP/s dense (%.3f ms per launch)\n",
         ops / (ms * 1e-3) / 1e12, ms / reps);
  CK(hipFree(out));
  return 0;
}
