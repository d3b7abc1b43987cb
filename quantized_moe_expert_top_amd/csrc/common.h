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
// The two constants of nibble_pairs() as register values: VOP3 takes no
// literal on gfx9, so with both constants folded the compiler splits every
// and-or into two instructions; held in registers, each is one v_and_or_b32.
// Create once per kernel (outside loops) and pass to nibble_pairs_r().
struct NibbleConsts {
  uint32_t mask, hi;
};
__device__ __forceinline__ NibbleConsts nibble_consts() {
  NibbleConsts k;
  asm volatile("v_mov_b32 %0, 0x000f000f" : "=v"(k.mask));
  asm volatile("s_mov_b32 %0, 0x43004300" : "=s"(k.hi));
  return k;
}
__device__ __forceinline__ void nibble_pairs_r(uint32_t w, const NibbleConsts& k, uint32_t& p0,
                                               uint32_t& p1, uint32_t& p2, uint32_t& p3) {
  p0 = (w & k.mask) | k.hi;
  p1 = ((w >> 4) & k.mask) | k.hi;
  p2 = ((w >> 8) & k.mask) | k.hi;
  p3 = ((w >> 12) & k.mask) | k.hi;
}
// bf16 pair (136, 136): 128 (bf16 exponent trick) + 8 (zero point); the codes
// of a zero weight widen to exactly this pattern.
constexpr uint32_t kBiasPair = 0x43084308u;

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// silu(g) * u = g * u / (1 + e^-g), with the hardware exp2 and reciprocal
// (about 1 ulp each). g -> -inf gives e^-g = inf and a zero reciprocal.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

template <typename T>
__device__ __forceinline__ T wave_shfl_xor(T v, int m) {
  return __shfl_xor(v, m, kWave);
}

// Top-k routing of one token by one wavefront ("Performance and verification",
// section "How it is verified": router ids are exact integer outputs).
// Each lane holds E/64 logits as 64-bit keys
//   key = orderable(logit) << 32 | (0xFFFFFFFF - expert)
// so the unsigned maximum is the largest logit with the lowest expert index on
// ties (+0.0 and -0.0 are made equal first). k rounds of a wave-wide max pick
// the experts in descending order; the owner lane clears the winner's key.
// The weights are a float32 softmax over the k selected logits. Lane j < k
// writes pick j to ids[j], w[j] (generic pointers: global memory or LDS).
__device__ __forceinline__ uint64_t route_key(float l, int e) {
  uint32_t b = __float_as_uint(l);
  if (b == 0x80000000u) b = 0u;  // -0.0 ties +0.0
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (static_cast<uint64_t>(ord) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(e));
}

// The logit a route_key() was built from (-0.0 comes back as +0.0, which it
// ties with).
__device__ __forceinline__ float route_key_logit(uint32_t ord) {
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

// Wave-wide max / sum through DPP (row_shr 1,2,4,8 inside 16-lane rows, then
// row_bcast 15/31 across rows) and a read of lane 63: a few cycles per step
// instead of an LDS permute per step. All 64 lanes must be active.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  v = mx(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x111, 0xf, 0xf, true)));
  v = mx(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x112, 0xf, 0xf, true)));
  v = mx(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x114, 0xf, 0xf, true)));
  v = mx(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x118, 0xf, 0xf, true)));
  v = mx(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x142, 0xa, 0xf, false)));
  v = mx(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x143, 0xc, 0xf, false)));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

template <int CTRL, int ROW_MASK, bool BOUND>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, BOUND));
}

__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32<0x111, 0xf, true>(v);
  v += dpp_f32<0x112, 0xf, true>(v);
  v += dpp_f32<0x114, 0xf, true>(v);
  v += dpp_f32<0x118, 0xf, true>(v);
  v += dpp_f32<0x142, 0xa, false>(v);
  v += dpp_f32<0x143, 0xc, false>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

template <int S>  // key slots per lane: E <= 64 * S
__device__ __forceinline__ void wave_topk(const float* __restrict__ row, int E, int k, int* ids,
                                          float* w) {
  const int lane = threadIdx.x & (kWave - 1);
  // every slot's logit is requested before any is used (slots past E read
  // the last logit and get key 0), so the row costs one memory round trip:
  // a guarded load per slot had compiled to S loads each waited on in turn
  float v[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int e = lane + kWave * s;
    v[s] = row[e < E ? e : E - 1];
  }
  uint64_t key[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int e = lane + kWave * s;
    key[s] = (e < E) ? route_key(v[s], e) : 0ull;  // valid keys are > 0
  }
  int my_e = 0;
  float my_l = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int s = 1; s < S; ++s) best = key[s] > best ? key[s] : best;
    // the 64-bit wave max as two 32-bit ones: the largest logit, then the
    // lowest expert index among the lanes holding it
    const uint32_t hi = static_cast<uint32_t>(best >> 32);
    const uint32_t mh = wave_max_u32(hi);
    const uint32_t ml = wave_max_u32(hi == mh ? static_cast<uint32_t>(best) : 0u);
    const uint64_t win = (static_cast<uint64_t>(mh) << 32) | ml;
#pragma unroll
    for (int s = 0; s < S; ++s)
      if (key[s] == win) key[s] = 0ull;
    if (lane == j) {
      my_e = static_cast<int>(0xFFFFFFFFu - ml);
      my_l = route_key_logit(mh);   // no reload of the row
    }
  }
  // softmax over the k picks; pick 0 holds the maximum
  const float lmax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_l), 0));
  const float z = (lane < k) ? expf(my_l - lmax) : 0.0f;
  const float sum = wave_sum_f32(z);
  if (lane < k) {
    ids[lane] = my_e;
    w[lane] = z / sum;
  }
}

// Raw buffer resource over [base, base + bytes) for buffer loads (untyped,
// 32-bit data format, no swizzle); loads at offsets past `bytes` return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}
typedef __attribute__((address_space(3))) void lds_void_t;

// 16-byte global load (global_load_dwordx4).
__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Block-wide exclusive scan of one int per thread for NTHR-thread blocks;
// `wave_tot` is an NTHR/64-int LDS scratch. Contains two barriers: call it
// from all threads of the block.
template <int NTHR>
__device__ __forceinline__ int block_excl_scan(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += o;
  }
  if (lane == kWave - 1) wave_tot[w] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < NTHR / kWave; ++i) {
    const int t = wave_tot[i];
    if (i < w) before += t;
    total += t;
  }
  __syncthreads();
  return before + incl - v;
}
__device__ __forceinline__ int block256_excl_scan(int v, int* wave_tot, int& total) {
  return block_excl_scan<256>(v, wave_tot, total);
}

}  // namespace moe
