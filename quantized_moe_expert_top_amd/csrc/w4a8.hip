// Grouped SwiGLU expert FFN, W4A8: int4 g128 weights (the W4A16 storage)
// against per-token int8 activations, on int8 MFMA.
//
// "Measured results", section "Speed": W4A8 beside W4A16 as a weight path.
//   1. quant: per row, s = absmax/127 (IEEE float32 division), codes
//      rint(x/s) clamped to [-127, 127]. The GEMM operand copy holds each
//      8-code chunk in the order {0,2,4,6,1,3,5,7} (the order the weight
//      unpacking below produces); the debug copy is in natural order.
//   2. gate/up: v_mfma_i32_32x32x32_i8 over (expert, 32- or 64-row,
//      128 h-column) tiles. A code c becomes the int8 16*(c - 8): the nibble
//      xor 8 (its two's complement 4-bit value) placed in the high half of a
//      byte, so the integer dot of a 128-k group is exact and needs no
//      zero-point correction; each group's dot is scaled by the group's fp16
//      scale (the tile's scales are staged in LDS) and accumulated in
//      float32; the epilogue applies row scale / 16 (exact) and SwiGLU,
//      writing h float32 in grouped order.
//   3. h quant: step 1 on h, one row per routed slot.
//   4. down: step 2 on hq against W2; y = hs/16 * acc, float32.
#include "common.h"
#include "launch.h"
#include "tiles.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kD = 3;       // 128-k groups in flight

// --------------------------------------------------------- quantization ----
__device__ __forceinline__ int quant_code4a8(float v, float s) {
  if (s == 0.0f) return 0;
  float q = rintf(v / s);
  q = fminf(fmaxf(q, -127.0f), 127.0f);
  return static_cast<int>(q);
}

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&v)[8]) {
  const uint4 w = ld16(p);
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16lo(u[i]);
    v[2 * i + 1] = bf16hi(u[i]);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// One wave per row of K values (bf16 x rows or float32 h rows), K % 128 == 0.
// Lane l takes 8-value chunks l, l + 64, ... A row of at most kRowChunks
// chunks per lane stays in registers between the absmax and the coding pass
// (one read of memory); longer rows are read twice.
constexpr int kRowChunks = 4;

__device__ __forceinline__ void code_chunk(const float (&v)[8], float s, int8_t* q, int8_t* dbg_q) {
  uint32_t nat[2] = {0, 0}, op[2] = {0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t b = static_cast<uint32_t>(quant_code4a8(v[i], s)) & 0xFFu;
    nat[i >> 2] |= b << (8 * (i & 3));
    op[i & 1] |= b << (8 * (i >> 1));   // even k in dword 0, odd k in dword 1
  }
  *reinterpret_cast<uint2*>(q) = make_uint2(op[0], op[1]);
  if (dbg_q) *reinterpret_cast<uint2*>(dbg_q) = make_uint2(nat[0], nat[1]);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void quant_rows_kernel(const T* __restrict__ src, int rows,
                                                              int K, int8_t* __restrict__ q,
                                                              float* __restrict__ scale,
                                                              int8_t* __restrict__ dbg_q,
                                                              float* __restrict__ dbg_s) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = blockIdx.x * (kThreads / kWave) + (threadIdx.x >> 6);
  if (r >= rows) return;  // uniform per wave
  const T* row = src + static_cast<size_t>(r) * K;
  const int C = K / 8;
  int8_t* qrow = q + static_cast<size_t>(r) * K;
  int8_t* drow = dbg_q ? dbg_q + static_cast<size_t>(r) * K : nullptr;
  float amax = 0.0f;
  if (C <= kRowChunks * kWave) {   // uniform: the row stays in registers
    float v[kRowChunks][8];
#pragma unroll
    for (int i = 0; i < kRowChunks; ++i) load8(row + min(lane + i * kWave, C - 1) * 8, v[i]);
#pragma unroll
    for (int i = 0; i < kRowChunks; ++i)
      if (lane + i * kWave < C)
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[i][j]));
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, wave_shfl_xor(amax, m));
    const float s = amax / 127.0f;
#pragma unroll
    for (int i = 0; i < kRowChunks; ++i) {
      const int c = lane + i * kWave;
      if (c < C) code_chunk(v[i], s, qrow + c * 8, drow ? drow + c * 8 : nullptr);
    }
    if (lane == 0) {
      scale[r] = s;
      if (dbg_s) dbg_s[r] = s;
    }
    return;
  }
  for (int c = lane; c < C; c += kWave) {
    float v[8];
    load8(row + c * 8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, wave_shfl_xor(amax, m));
  const float s = amax / 127.0f;
  for (int c = lane; c < C; c += kWave) {
    float v[8];
    load8(row + c * 8, v);
    code_chunk(v, s, qrow + c * 8, drow ? drow + c * 8 : nullptr);
  }
  if (lane == 0) {
    scale[r] = s;
    if (dbg_s) dbg_s[r] = s;
  }
}

// ------------------------------------------------------------- int8 GEMM ----
// KIND 0: gate/up. Wave w owns h-columns [nt*128 + 32w, +32): B subtile 0 the
//         gate rows, subtile 1 the matching up rows. Out: h float32 [R, I].
// KIND 1: down. Wave w owns W2 rows [nt*256 + 64w, +64) as two subtiles.
// K order inside a 128-k group: lane half hf takes k = 64*hf + [0, 64); MFMA
// step s (of 4) takes k = 64*hf + 16*s + [0, 16) for that half, on both
// operands, whose 16 bytes hold those k in the order {0,2,4,6,1,3,5,7,
// 8,10,12,14,9,11,13,15} (the activation codes are stored that way; the
// weight unpacking yields it).
// Per group: codes of the group (32 bytes per lane and subtile) and the raw
// fp16 scales stream through a register ring of kD groups, with this thread's
// 16-byte share of the activation tile; the activation tile is written to a
// swizzled LDS stage one step before use (two stages).
template <int KIND, int MT>
__global__ __launch_bounds__(kThreads, 2) void w4a8_mfma_kernel(
    const int8_t* __restrict__ A, const float* __restrict__ a_scale,
    const uint8_t* __restrict__ W, const uint16_t* __restrict__ S, const int* __restrict__ offsets,
    const int* __restrict__ sorted_slot, float* __restrict__ out, int K, int N, int E, int topk,
    int NT) {
  constexpr int BM = 32 * MT;        // tile rows: MT m-subtiles of 32 share each B fragment
  constexpr int STAGE = BM * 128;    // bytes of one activation stage
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[2 * STAGE];
  // per wave: one group's codes of its two 32-row B subtiles (64 bytes a row)
  __shared__ __attribute__((aligned(16))) uint8_t b_lds[kThreads / kWave][2 * 32 * 64];
  __shared__ int row_src[BM];
  __shared__ float row_scale[BM];
  __shared__ int sm_pref[kThreads / kWave];
  __shared__ int sm_out[5];
  extern __shared__ __attribute__((aligned(16))) uint16_t s_lds[];  // [256][G]: fp16 scales of the tile's weight rows

  TileInfo ti;
  if (!find_tile<BM>(offsets, E, NT, sm_pref, sm_out, ti)) return;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int G = K / kGroup;

  // whether this lane's B columns exist (two subtiles)
  bool nvalid[2];
  if (KIND == 0) {
    const int n = ti.nt * 128 + wv * 32 + l32;  // h column
    nvalid[0] = nvalid[1] = n < N / 2;
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) nvalid[j] = ti.nt * 256 + wv * 64 + j * 32 + l32 < N;
  }
  const uint32_t rowb = static_cast<uint32_t>(K / 2);
  const __amdgpu_buffer_rsrc_t w_rsrc =
      buffer_rsrc(W + static_cast<size_t>(ti.e) * N * rowb, static_cast<uint32_t>(N) * rowb);
  const __amdgpu_buffer_rsrc_t s_rsrc =
      buffer_rsrc(S + static_cast<size_t>(ti.e) * N * G, static_cast<uint32_t>(N * G) * 2u);
  // Codes are fetched row-contiguous: a wave instruction reads 16 rows x 64
  // bytes (four lanes a row, one 16-byte chunk each), rows 0-15 of a subtile
  // in one load and rows 16-31 in the next. Compute moves them through the
  // wave's LDS area into the MFMA operand layout. Rows past the expert read
  // as zeros (or as the up rows, for a gate tile past I); their columns are
  // dropped.
  uint32_t woff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row0 = (KIND == 0) ? j * (N / 2) + ti.nt * 128 + wv * 32 : ti.nt * 256 + wv * 64 + j * 32;
    woff[j] = static_cast<uint32_t>(row0 + (lane >> 2)) * rowb + (lane & 3) * 16;
  }
  // this lane's rows within the tile's 256 scale rows
  int srow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) srow[j] = (KIND == 0) ? j * 128 + wv * 32 + l32 : wv * 64 + j * 32 + l32;

  // The scales of the tile's 256 weight rows are contiguous runs of S (two
  // 128-row strips, gate and up, or one 256-row strip) starting at multiples
  // of 256 bytes: they are copied to LDS in 16-byte chunks (a per-group load
  // of one fp16 per row would touch 32 rows per instruction). Rows past the
  // expert read as 0 through the buffer resource and are never used. Loads
  // and stores are unconditional (clamped) so all stay in flight together.
  constexpr int kScBatch = 4;
  const int sc_chunks = 32 * G;           // 256 rows * G * 2 bytes / 16
  const uint32_t strip0 = static_cast<uint32_t>((KIND == 0 ? ti.nt * 128 : ti.nt * 256) * G * 2);
  const uint32_t strip1 = static_cast<uint32_t>((N / 2 + ti.nt * 128) * G * 2);
  uint4 scv[kScBatch];
  auto sc_src = [&](int i) -> uint32_t {
    if (KIND == 0 && i >= 16 * G) return strip1 + (i - 16 * G) * 16;
    return strip0 + i * 16;
  };
#pragma unroll
  for (int u = 0; u < kScBatch; ++u)
    scv[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           s_rsrc, sc_src(min(u * kThreads + tid, sc_chunks - 1)), 0, 0));

  struct Grp {
    uint4 q[2][2];
    uint4 a[MT];
  };
  Grp ring[kD];
  auto issue_w = [&](int g, Grp& b) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      b.q[j][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                w_rsrc, woff[j], g * 64, 0));
      b.q[j][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                w_rsrc, woff[j] + 16 * rowb, g * 64, 0));
    }
  };
  // the weight strip does not depend on the rows: start streaming it first
#pragma unroll
  for (int d = 0; d < kD - 1; ++d) issue_w(min(d, G - 1), ring[d]);

  int my_src = 0;
  if (tid < BM) {
    const int p = ti.p_begin + tid;
    const int pv = p < ti.p_end ? p : ti.p_begin;
    my_src = (KIND == 0) ? sorted_slot[pv] / topk : pv;
    row_src[tid] = my_src;
  }
  __syncthreads();
  // the row scale is needed only by the epilogue: its load overlaps the
  // first activation loads
  float my_scale = 0.0f;
  if (tid < BM) my_scale = a_scale[my_src];
  // this thread's activation chunks: slot L = tid + 256 i of a stage holds
  // row L/8, 16-byte chunk (L%8) ^ ((row/2)%8); the xor term is the same for
  // rows 32 apart
  const int arow = tid >> 3, achunk = ((tid & 7) ^ ((arow >> 1) & 7)) * 16;
  const int8_t* asrc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
    asrc[i] = A + static_cast<size_t>(row_src[arow + 32 * i]) * K + achunk;
  const int adst = tid * 16;
#pragma unroll
  for (int d = 0; d < kD - 1; ++d)
#pragma unroll
    for (int i = 0; i < MT; ++i) ring[d].a[i] = ld16(asrc[i] + min(d, G - 1) * kGroup);

  // LDS offsets of this lane's A operand for the 4 MFMA steps of a group
  // (m-subtile i adds 32 rows = 4096 bytes)
  int aoffs[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) aoffs[s] = (l32 * 8 + ((hf * 4 + s) ^ ((l32 >> 1) & 7))) * 16;

  auto issue = [&](int g, Grp& b) {
    issue_w(g, b);
#pragma unroll
    for (int i = 0; i < MT; ++i) b.a[i] = ld16(asrc[i] + g * kGroup);
  };
  auto stage_a = [&](const Grp& b, int stage) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
      *reinterpret_cast<uint4*>(a_lds + stage * STAGE + i * 4096 + adst) = b.a[i];
  };

  float acc[MT][2][16];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // 8 codes (one dword, byte b = k(2b) | k(2b+1) << 4) -> 8 int8 holding
  // 16 * (code - 8): e = {k0, k2, k4, k6}, o = {k1, k3, k5, k7}
  const uint32_t kFlip = 0x88888888u, kHiN = 0xF0F0F0F0u;
  auto unpack = [&](uint32_t w, uint32_t& e, uint32_t& o) {
    const uint32_t f = w ^ kFlip;
    e = (f << 4) & kHiN;
    o = f & kHiN;
  };
  auto compute = [&](const Grp& b, int stage, int g) {
    const uint8_t* st = a_lds + stage * STAGE;
    // the group's codes into the operand layout: lane (l32, hf) takes bytes
    // [32 hf, +32) of row l32. Slot (row, chunk c) sits at row * 4 +
    // (c ^ (row / 4 % 4)), so both the writes (16 rows x 4 chunks) and the
    // reads (32 rows, one chunk each) hit distinct banks. The wave's LDS
    // operations complete in order, so no wait or barrier is needed.
    uint8_t* bw = b_lds[wv];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = h * 16 + (lane >> 2), c = lane & 3;
        *reinterpret_cast<uint4*>(bw + j * 2048 + (row * 4 + (c ^ ((row >> 2) & 3))) * 16) = b.q[j][h];
      }
    uint4 bq[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int c = 2 * hf + t;
        bq[j][t] = *reinterpret_cast<const uint4*>(bw + j * 2048 + (l32 * 4 + (c ^ ((l32 >> 2) & 3))) * 16);
      }
    uint4 av[MT][4];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        av[i][s] = *reinterpret_cast<const uint4*>(st + i * 4096 + aoffs[s]);
    uint16_t sc_bits[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) sc_bits[j] = s_lds[srow[j] * G + g];
    __builtin_amdgcn_sched_barrier(0);
    i32x16_t accg[MT][2];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) accg[i][j][r] = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        // step s uses bytes [8s, 8s + 8) of the lane's 32 code bytes
        const uint32_t w0 = (&bq[j][s >> 1].x)[(s & 1) * 2];
        const uint32_t w1 = (&bq[j][s >> 1].x)[(s & 1) * 2 + 1];
        uint32_t e0, o0, e1, o1;
        unpack(w0, e0, o0);
        unpack(w1, e1, o1);
        i32x4_t bop;
        bop[0] = static_cast<int>(e0);
        bop[1] = static_cast<int>(o0);
        bop[2] = static_cast<int>(e1);
        bop[3] = static_cast<int>(o1);
#pragma unroll
        for (int i = 0; i < MT; ++i)
          accg[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
              __builtin_bit_cast(i32x4_t, av[i][s]), bop, accg[i][j], 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float sc = fp16_bits_to_f32(sc_bits[j]);
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] += sc * static_cast<float>(accg[i][j][r]);
    }
  };

  // scale strips into LDS (read after the loop's first barrier)
  for (int i0 = 0; i0 < sc_chunks; i0 += kScBatch * kThreads) {
    if (i0 > 0) {
#pragma unroll
      for (int u = 0; u < kScBatch; ++u)
        scv[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                               s_rsrc, sc_src(min(i0 + u * kThreads + tid, sc_chunks - 1)), 0, 0));
    }
#pragma unroll
    for (int u = 0; u < kScBatch; ++u)
      *reinterpret_cast<uint4*>(s_lds + min(i0 + u * kThreads + tid, sc_chunks - 1) * 8) = scv[u];
  }
  asm volatile("" ::"s"(out));
  stage_a(ring[0], 0);
  if (tid < BM) row_scale[tid] = my_scale;   // read after the loop's barriers
  for (int g0 = 0; g0 < G; g0 += kD) {
#pragma unroll
    for (int d = 0; d < kD; ++d) {
      const int g = g0 + d;
      __syncthreads();  // group g's stage is written; group g + 1's is free
      issue(min(g + kD - 1, G - 1), ring[(d + kD - 1) % kD]);
      if (g < G) compute(ring[d], g & 1, g);
      if (g + 1 < G) stage_a(ring[(d + 1) % kD], (g + 1) & 1);
    }
  }

  // epilogue; C layout: lane holds column l32, rows 8*(r/4) + 4*hf + (r%4).
  // Stores go through a buffer resource based at the tile's first row and
  // column, at 32-bit offsets: rows past the expert's block lie past the
  // resource's end, columns past the row width are sent there, and the
  // hardware drops both (no branch per element).
  constexpr uint32_t kPastEnd = 0x80000000u;
  const int ow = (KIND == 0) ? N / 2 : N;
  const int cb = (KIND == 0) ? ti.nt * 128 : ti.nt * 256;
  const int rows = min(ti.p_end - ti.p_begin, 32 * MT);
  const uint32_t orowb = static_cast<uint32_t>(ow) * 4;
  const __amdgpu_buffer_rsrc_t o_rsrc =
      buffer_rsrc(out + static_cast<size_t>(ti.p_begin) * ow + cb,
                  static_cast<uint32_t>(rows - 1) * orowb + static_cast<uint32_t>(ow - cb) * 4);
  uint32_t coff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = (KIND == 0) ? wv * 32 + l32 : wv * 64 + j * 32 + l32;
    coff[j] = nvalid[j] ? static_cast<uint32_t>(hf * 4) * orowb + c * 4 : kPastEnd;
  }
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 32 * i + (r >> 2) * 8 + hf * 4 + (r & 3);
      const uint32_t roff = static_cast<uint32_t>(m - hf * 4) * orowb;
      const float rs = row_scale[m] * 0.0625f;   // the operand codes carry a factor 16
      if (KIND == 0) {
        const float v = silu_mul(acc[i][0][r] * rs, acc[i][1][r] * rs);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), o_rsrc,
                                              coff[0] + roff, 0, 0);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float v = acc[i][j][r] * rs;
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), o_rsrc,
                                                coff[j] + roff, 0, 0);
        }
      }
    }
}

// Tile rows: 64 (MT = 2) once the routed rows average a full 32-row tile per
// active expert, so each expert's weight strip is streamed fewer times.
template <int KIND>
hipError_t launch_w4a8_gemm(const int8_t* A, const float* a_scale, const uint8_t* W,
                            const uint16_t* S, const int* offsets, const int* sorted_slot,
                            float* out, int K, int N, int E, int topk, int T, hipStream_t s) {
  const int NT = (KIND == 0) ? (N / 2 + 127) / 128 : (N + 255) / 256;
  const long long R = static_cast<long long>(T) * topk;
  const long long act = R < E ? R : E;
  const bool wide = R >= 32 * act;
  const int BM = wide ? 64 : 32;
  const long long mt_up = (R + BM - 1) / BM + act;
  const dim3 grid(static_cast<unsigned>((mt_up * NT + 7) / 8 * 8));
  const size_t lds = static_cast<size_t>(256) * (K / kGroup) * 2;   // the tile's scale strips
  if (wide)
    hipLaunchKernelGGL((w4a8_mfma_kernel<KIND, 2>), grid, dim3(kThreads), lds, s, A, a_scale, W,
                       S, offsets, sorted_slot, out, K, N, E, topk, NT);
  else
    hipLaunchKernelGGL((w4a8_mfma_kernel<KIND, 1>), grid, dim3(kThreads), lds, s, A, a_scale, W,
                       S, offsets, sorted_slot, out, K, N, E, topk, NT);
  return hipGetLastError();
}

struct W4A8Ws {
  int8_t* xq;
  float* xs;
  float* h;
  int8_t* hq;
  float* hs;
};

W4A8Ws carve(void* ws, int T, int H, int I, int k) {
  const size_t R = static_cast<size_t>(T) * k;
  char* p = static_cast<char*>(ws);
  W4A8Ws w;
  w.xq = reinterpret_cast<int8_t*>(p);
  p += align_up(static_cast<size_t>(T) * H, 256);
  w.xs = reinterpret_cast<float*>(p);
  p += align_up(static_cast<size_t>(T) * 4, 256);
  w.h = reinterpret_cast<float*>(p);
  p += align_up(R * I * 4, 256);
  w.hq = reinterpret_cast<int8_t*>(p);
  p += align_up(R * I, 256);
  w.hs = reinterpret_cast<float*>(p);
  return w;
}

}  // namespace

size_t w4a8_workspace_bytes(int T, int H, int I, int, int k) {
  const size_t R = static_cast<size_t>(T) * k;
  return align_up(static_cast<size_t>(T) * H, 256) + align_up(static_cast<size_t>(T) * 4, 256) +
         align_up(R * I * 4, 256) + align_up(R * I, 256) + align_up(R * 4, 256);
}

hipError_t launch_w4a8_ffn(int T, int H, int I, int E, int k, const uint16_t* x,
                           const uint8_t* w13, const uint16_t* s13, const uint8_t* w2,
                           const uint16_t* s2, const int* offsets, const int* sorted_slot,
                           float* y, const W4A8Debug& dbg, void* ws, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const W4A8Ws w = carve(ws, T, H, I, k);
  const int R = T * k;
  const int rpb = kThreads / kWave;
  quant_rows_kernel<uint16_t><<<(T + rpb - 1) / rpb, kThreads, 0, s>>>(x, T, H, w.xq, w.xs,
                                                                       dbg.xq, dbg.xs);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  err = launch_w4a8_gemm<0>(w.xq, w.xs, w13, s13, offsets, sorted_slot, w.h, H, 2 * I, E, k,
                            T, s);
  if (err != hipSuccess) return err;
  quant_rows_kernel<float><<<(R + rpb - 1) / rpb, kThreads, 0, s>>>(w.h, R, I, w.hq, w.hs,
                                                                    dbg.hq, dbg.hs);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_w4a8_gemm<1>(w.hq, w.hs, w2, s2, offsets, sorted_slot, y, I, H, E, k, T, s);
}

}  // namespace moe
