// Device helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;
constexpr int kGroup = 128;  // int4 scale group along K

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(int)))) int i32x16_t;

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest even (native v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fp16_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// 8 bf16 (one 16-byte chunk, natural k order a = {x0x1, x2x3, x4x5, x6x7}) ->
// the pair order produced by nibble_pairs(): {x0x4, x1x5, x2x6, x3x7}.
__device__ __forceinline__ uint4 pair_permute(uint4 a) {
  uint4 o;
  o.x = (a.x & 0xFFFFu) | (a.z << 16);
  o.y = (a.x >> 16) | (a.z & 0xFFFF0000u);
  o.z = (a.y & 0xFFFFu) | (a.w << 16);
  o.w = (a.y >> 16) | (a.w & 0xFFFF0000u);
  return o;
}

// One dword of packed int4 codes (byte b = k(2b) | k(2b+1) << 4) -> four bf16
// pairs holding 128 + q exactly (bf16 0x43XX with the code in the low mantissa
// bits): {k0,k4}, {k1,k5}, {k2,k6}, {k3,k7}. The caller subtracts the
// 128 + 8 bias through the per-chunk sum of its activations.
__device__ __forceinline__ void nibble_pairs(uint32_t w, uint32_t& p0, uint32_t& p1,
                                             uint32_t& p2, uint32_t& p3) {
  constexpr uint32_t kMask = 0x000F000Fu, kHi = 0x43004300u;
  p0 = (w & kMask) | kHi;
  p1 = ((w >> 4) & kMask) | kHi;
  p2 = ((w >> 8) & kMask) | kHi;
  p3 = ((w >> 12) & kMask) | kHi;
}
// bf16 pair (136, 136): 128 (bf16 exponent trick) + 8 (zero point); the codes
// of a zero weight widen to exactly this pattern.
constexpr uint32_t kBiasPair = 0x43084308u;

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + expf(-g)) * u;
}

template <typename T>
__device__ __forceinline__ T wave_shfl_xor(T v, int m) {
  return __shfl_xor(v, m, kWave);
}

// Non-temporal-free 16-byte global load (plain; the compiler emits
// global_load_dwordx4).
__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

}  // namespace moe
