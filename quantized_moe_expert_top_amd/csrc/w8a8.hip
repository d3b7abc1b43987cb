// Grouped SwiGLU expert FFN on int8 x int8 -> int32 MFMA (W8A8).
//
// "Performance and verification", section "Why it is fast": routed experts of
// a prompt run as grouped int8 tensor-core GEMMs. Here:
//   1. act_quant: per token row, s = absmax/127 (IEEE float32 division), codes
//      rint(x/s) clamped to [-127, 127] (round half to even).
//   2. gate/up: v_mfma_i32_32x32x32_i8 over (expert, 128-row, 128-column) tiles;
//      the epilogue dequantizes (acc * xs[t] * s13[e,n]) and applies SwiGLU in
//      float32, writing h (float32) in grouped order.
//   3. h_quant: the same per-row rule on h (one row per routed slot). h stays
//      float32 until here so the code decisions match a float32 reference.
//   4. down: int8 MFMA over (expert, 128-row, 256-column) tiles; y = acc *
//      hs[p] * s2[e,n], stored float32.
// The int32 accumulators are exact, so they are reproducible bit for bit.
#include "common.h"
#include "launch.h"
#include "tiles.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// --------------------------------------------------------- quantization ----
__device__ __forceinline__ int8_t quant_code(float v, float s) {
  if (s == 0.0f) return 0;
  float q = rintf(v / s);
  q = fminf(fmaxf(q, -127.0f), 127.0f);
  return static_cast<int8_t>(static_cast<int>(q));
}

// One wave per token row of x (bf16 [T, H]); H % 8 == 0.
// One wave per row. A row of at most kRowChunks chunks per lane stays in
// registers between the absmax and the coding pass (one read of memory);
// longer rows are read twice.
constexpr int kRowChunks = 4;

__device__ __forceinline__ uint2 code_bf16x8(const uint4& v, float s) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t packed[2] = {0, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = static_cast<uint8_t>(quant_code(bf16lo(w[i]), s));
    const uint32_t hi = static_cast<uint8_t>(quant_code(bf16hi(w[i]), s));
    packed[i >> 1] |= (lo | (hi << 8)) << (16 * (i & 1));
  }
  return make_uint2(packed[0], packed[1]);
}
__device__ __forceinline__ float amax_bf16x8(const uint4& v, float amax) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fmaxf(fabsf(bf16lo(w[i])), fabsf(bf16hi(w[i]))));
  return amax;
}
__device__ __forceinline__ uint32_t code_f32x4(const float4& v, float s) {
  return static_cast<uint8_t>(quant_code(v.x, s)) |
         (static_cast<uint32_t>(static_cast<uint8_t>(quant_code(v.y, s))) << 8) |
         (static_cast<uint32_t>(static_cast<uint8_t>(quant_code(v.z, s))) << 16) |
         (static_cast<uint32_t>(static_cast<uint8_t>(quant_code(v.w, s))) << 24);
}
__device__ __forceinline__ float amax_f32x4(const float4& v, float amax) {
  return fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
}

__global__ __launch_bounds__(kThreads) void act_quant_kernel(const uint16_t* __restrict__ x,
                                                             int T, int H,
                                                             int8_t* __restrict__ xq,
                                                             float* __restrict__ xs,
                                                             int8_t* __restrict__ dbg_xq,
                                                             float* __restrict__ dbg_xs) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (kThreads / kWave) + (threadIdx.x >> 6);
  if (t >= T) return;
  const uint16_t* row = x + static_cast<size_t>(t) * H;
  int8_t* qrow = xq + static_cast<size_t>(t) * H;
  int8_t* drow = dbg_xq ? dbg_xq + static_cast<size_t>(t) * H : nullptr;
  const int C = H / 8;   // 16-byte chunks of 8 values
  float amax = 0.0f;
  if (C <= kRowChunks * kWave) {   // uniform: the row stays in registers
    uint4 v[kRowChunks];
#pragma unroll
    for (int i = 0; i < kRowChunks; ++i) v[i] = ld16(row + min(lane + i * kWave, C - 1) * 8);
#pragma unroll
    for (int i = 0; i < kRowChunks; ++i)
      if (lane + i * kWave < C) amax = amax_bf16x8(v[i], amax);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, wave_shfl_xor(amax, m));
    const float s = amax / 127.0f;
#pragma unroll
    for (int i = 0; i < kRowChunks; ++i) {
      const int c = lane + i * kWave;
      if (c < C) {
        const uint2 pv = code_bf16x8(v[i], s);
        *reinterpret_cast<uint2*>(qrow + c * 8) = pv;
        if (drow) *reinterpret_cast<uint2*>(drow + c * 8) = pv;
      }
    }
    if (lane == 0) {
      xs[t] = s;
      if (dbg_xs) dbg_xs[t] = s;
    }
    return;
  }
  for (int c = lane; c < C; c += kWave) amax = amax_bf16x8(ld16(row + c * 8), amax);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, wave_shfl_xor(amax, m));
  const float s = amax / 127.0f;
  for (int c = lane; c < C; c += kWave) {
    const uint2 pv = code_bf16x8(ld16(row + c * 8), s);
    *reinterpret_cast<uint2*>(qrow + c * 8) = pv;
    if (drow) *reinterpret_cast<uint2*>(drow + c * 8) = pv;
  }
  if (lane == 0) {
    xs[t] = s;
    if (dbg_xs) dbg_xs[t] = s;
  }
}

__global__ __launch_bounds__(kThreads) void h_quant_kernel(const float* __restrict__ h, int R,
                                                           int I, int8_t* __restrict__ hq,
                                                           float* __restrict__ hs,
                                                           int8_t* __restrict__ dbg_hq,
                                                           float* __restrict__ dbg_hs) {
  const int lane = threadIdx.x & (kWave - 1);
  const int p = blockIdx.x * (kThreads / kWave) + (threadIdx.x >> 6);
  if (p >= R) return;
  const float* row = h + static_cast<size_t>(p) * I;
  int8_t* qrow = hq + static_cast<size_t>(p) * I;
  int8_t* drow = dbg_hq ? dbg_hq + static_cast<size_t>(p) * I : nullptr;
  const int C = I / 4;   // 16-byte chunks of 4 values
  float amax = 0.0f;
  if (C <= kRowChunks * kWave) {   // uniform: the row stays in registers
    float4 v[kRowChunks];
#pragma unroll
    for (int i = 0; i < kRowChunks; ++i)
      v[i] = *reinterpret_cast<const float4*>(row + min(lane + i * kWave, C - 1) * 4);
#pragma unroll
    for (int i = 0; i < kRowChunks; ++i)
      if (lane + i * kWave < C) amax = amax_f32x4(v[i], amax);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, wave_shfl_xor(amax, m));
    const float s = amax / 127.0f;
#pragma unroll
    for (int i = 0; i < kRowChunks; ++i) {
      const int c = lane + i * kWave;
      if (c < C) {
        const uint32_t q = code_f32x4(v[i], s);
        *reinterpret_cast<uint32_t*>(qrow + c * 4) = q;
        if (drow) *reinterpret_cast<uint32_t*>(drow + c * 4) = q;
      }
    }
    if (lane == 0) {
      hs[p] = s;
      if (dbg_hs) dbg_hs[p] = s;
    }
    return;
  }
  for (int c = lane; c < C; c += kWave)
    amax = amax_f32x4(*reinterpret_cast<const float4*>(row + c * 4), amax);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, wave_shfl_xor(amax, m));
  const float s = amax / 127.0f;
  for (int c = lane; c < C; c += kWave) {
    const uint32_t q = code_f32x4(*reinterpret_cast<const float4*>(row + c * 4), s);
    *reinterpret_cast<uint32_t*>(qrow + c * 4) = q;
    if (drow) *reinterpret_cast<uint32_t*>(drow + c * 4) = q;
  }
  if (lane == 0) {
    hs[p] = s;
    if (dbg_hs) dbg_hs[p] = s;
  }
}

// ------------------------------------------------------------- int8 GEMM ----
// Tiles of BM rows x 256 B rows. A block has WM x WN waves; wave (wm, wn) owns
// BM/WM tile rows and 256/WN B rows as 32 x 32 MFMA subtiles (MI x NJ).
// KIND 0: gate/up. Tile = BM rows x 128 h-columns: the B tile holds the 128
//         gate rows and the 128 matching up rows (256 W13 rows). Wave wn owns
//         h-columns [wn*128/WN, +128/WN): its first NJ/2 subtiles are those
//         gate rows, the last NJ/2 the matching up rows. Out: h float32 [R, I].
// KIND 1: down. Tile = BM rows x 256 W2 rows; wave wn owns W2 rows
//         [wn*256/WN, +256/WN). Out: y float32 [R, H].
// Pipeline: K advances in BK-byte stages; kStages stages rotate through LDS,
// each moved HBM -> LDS by buffer_load_dwordx4 ... lds (no register staging;
// the buffer form, unlike the global one, leaves LDS reads countable in order,
// so operand reads overlap the MFMAs). A wave instruction fills 64
// consecutive 16-byte LDS slots; slot s of a tile holds row s/CPR, chunk
// (s%CPR) ^ swizzle(row), so each row's BK bytes are still read as one
// coalesced run while the MFMA operand reads (32 rows, one chunk each) hit
// distinct LDS banks. Waits are explicit (vmcnt + barrier) so loads of later
// stages stay in flight across the barrier: each stage is exactly
// kLoadsPerStage vector-memory instructions per thread and nothing else in
// the loop touches vector memory (the library build rejects any kernel that
// spills to scratch, which would add such instructions).
// MFMA operand k order inside one 32-k step: lane half hf = lane/32 takes
// k = 32*ks + 16*hf + [0, 16).
constexpr int kW8BN = 256;                       // B rows per tile

template <int BM_, int WM_, int WN_, int BK_, int STAGES_, int BPC_>
struct W8Geom {
  static constexpr int BM = BM_, WM = WM_, WN = WN_, BK = BK_;
  static constexpr int kStages = STAGES_;
  static constexpr int kThreads = WM * WN * kWave;
  static constexpr int kCPR = BK / 16;                          // 16-byte chunks of a row per stage
  static constexpr int kMI = BM / WM / 32;                      // 32-row subtiles per wave
  static constexpr int kNJ = kW8BN / WN / 32;                   // 32-column subtiles per wave
  static constexpr int kASlots = BM * kCPR;                     // 16-byte A slots per stage
  static constexpr int kBSlots = kW8BN * kCPR;
  static constexpr int kStageBytes = (kASlots + kBSlots) * 16;
  static constexpr int kAPer = kASlots / kThreads;              // A loads per thread per stage
  static constexpr int kBPer = kBSlots / kThreads;
  static constexpr int kLoadsPerStage = kAPer + kBPer;
  static constexpr int kBlocksPerCU = BPC_;
  static_assert(kASlots % kThreads == 0 && kBSlots % kThreads == 0, "slots split evenly");
  static_assert(kMI >= 1 && kNJ >= 2 && kNJ % 2 == 0 && kNJ <= 4, "wave tile shape");
  static_assert(kAPer <= 8 && kBPer <= 8, "slot arrays hold eight per thread");
  // dynamic stages plus about 4 KB of static arrays per block
  static_assert(kBlocksPerCU * (kStages * kStageBytes + 4096) <= 160 * 1024, "LDS per CU");
};
// four waves, 64-byte stages, two blocks per CU. Measured against it at
// T 4096 (same box): eight waves with 128-byte stages at one block per CU
// (each row's stage one whole cache line) ran the FFN 4% slower, and the same
// with stages staged through registers (three or four in flight per thread)
// 12% and 40% slower.
using W8Tile = W8Geom<128, 2, 2, 64, 3, 2>;

// LDS slot of (row, chunk c) in a stage: rows of CPR chunks, the chunk index
// XOR-swizzled by the row so that 16 consecutive rows read at one chunk fall
// in distinct banks (4 banks per 16-byte chunk, 64 banks)
template <int CPR>
__device__ __forceinline__ int swz_bits(int row) { return (row / (16 / CPR)) & (CPR - 1); }
template <int CPR>
__device__ __forceinline__ int swz(int row, int c) { return row * CPR + (c ^ swz_bits<CPR>(row)); }

// s_waitcnt vmcnt(N) then s_barrier, for the counts the pipeline uses
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N == 0 || N == 3 || N == 4 || N == 6 || N == 8 || N == 9 || N == 12 || N == 16,
                "add the count here");
  if constexpr (N == 16) asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 12) asm volatile("s_waitcnt vmcnt(12)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 9) asm volatile("s_waitcnt vmcnt(9)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 6) asm volatile("s_waitcnt vmcnt(6)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 3) asm volatile("s_waitcnt vmcnt(3)\n\ts_barrier" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}
// wait until a stage has landed while `later` later stages (of LPS loads
// each) may still be in flight, then barrier; later <= MAXL
template <int LPS, int MAXL>
__device__ __forceinline__ void wait_stage(int later) {
  if constexpr (MAXL >= 4) { if (later >= 4) { wait_vm_barrier<4 * LPS>(); return; } }
  if constexpr (MAXL >= 3) { if (later == 3) { wait_vm_barrier<3 * LPS>(); return; } }
  if constexpr (MAXL >= 2) { if (later == 2) { wait_vm_barrier<2 * LPS>(); return; } }
  if constexpr (MAXL >= 1) { if (later == 1) { wait_vm_barrier<LPS>(); return; } }
  wait_vm_barrier<0>();
}

template <int KIND, class G>
__global__ __launch_bounds__(G::kThreads, G::kBlocksPerCU) void w8a8_mfma_kernel(
    const int8_t* __restrict__ A, const float* __restrict__ a_scale,
    const int8_t* __restrict__ W, const float* __restrict__ w_scale,
    const int* __restrict__ offsets, const int* __restrict__ sorted_slot, int a_rows, int K,
    int N, int E, int topk, int NT, float* __restrict__ h_out, float* __restrict__ y_out,
    int32_t* __restrict__ dbg_acc) {
  constexpr int BM = G::BM, MI = G::kMI, NJ = G::kNJ, NTHR = G::kThreads;
  constexpr int BK = G::BK, CPR = G::kCPR, STAGES = G::kStages;
  constexpr int RW = BM / G::WM;        // tile rows per wave
  constexpr int HCW = 128 / G::WN;      // h-columns per wave (gate/up)
  constexpr int BW = kW8BN / G::WN;     // B rows per wave (down)
  extern __shared__ __attribute__((aligned(16))) uint8_t w8_lds[];  // STAGES * kStageBytes
  __shared__ int row_src[BM];
  __shared__ __attribute__((aligned(16))) float row_scale[BM];  // activation scale of each tile row
  __shared__ float col_scale[kW8BN];  // weight scale of each B tile row
  __shared__ int sm_pref[NTHR / kWave];
  __shared__ int sm_out[5];

  TileInfo ti;
  if (!find_tile<BM, NTHR>(offsets, E, NT, sm_pref, sm_out, ti)) return;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int wm = wv / G::WN, wn = wv % G::WN;   // wave's row band and B band
  const int I = N / 2;  // KIND 0 only

  // W row held at B tile row j (0..255)
  auto b_row = [&](int j) -> int {
    if (KIND == 0) {
      const int half = j >> 7, c = ti.nt * 128 + (j & 127);
      return half * I + (c < I ? c : I - 1);
    }
    const int r = ti.nt * kW8BN + j;
    return r < N ? r : N - 1;
  };
  // B tile row of this lane in the wave's subtile j
  auto b_tile_row = [&](int j) -> int {
    if (KIND == 0) return (j / (NJ / 2)) * 128 + wn * HCW + (j % (NJ / 2)) * 32 + l32;
    return wn * BW + j * 32 + l32;
  };
  // source row of each A tile row (token for gate/up, grouped row for down);
  // rows past the expert's block read the tile's first row (results dropped).
  // The scales the epilogue needs are staged here, off its critical path.
  for (int r = tid; r < BM; r += NTHR) {
    const int p = ti.p_begin + r;
    const int pv = (p < ti.p_end) ? p : ti.p_begin;
    const int src = (KIND == 0) ? sorted_slot[pv] / topk : pv;
    row_src[r] = src;
    row_scale[r] = a_scale[src];
  }
  for (int j = tid; j < kW8BN; j += NTHR)
    col_scale[j] = w_scale[static_cast<size_t>(ti.e) * N + b_row(j)];
  __syncthreads();

  // this thread's A and B slots per stage (slot = wave * 64 + lane + NTHR * v),
  // as byte offsets into buffer resources over A and this expert's W rows
  const __amdgpu_buffer_rsrc_t a_rsrc = buffer_rsrc(A, static_cast<uint32_t>(a_rows) * K);
  const __amdgpu_buffer_rsrc_t b_rsrc =
      buffer_rsrc(W + static_cast<size_t>(ti.e) * N * K, static_cast<uint32_t>(N) * K);
  // fixed-size arrays: a lambda capturing arrays whose size depends on the
  // template parameters makes the host pass drop the kernel's launch stub
  uint32_t aoff[8], boff[8], akc[8], bkc[8];   // row offset + chunk, and the chunk's k
#pragma unroll
  for (int v = 0; v < G::kAPer; ++v) {
    const int s = tid + NTHR * v, row = s / CPR, c = (s % CPR) ^ swz_bits<CPR>(row);
    aoff[v] = static_cast<uint32_t>(row_src[row]) * K + c * 16;
    akc[v] = c * 16;
  }
#pragma unroll
  for (int v = 0; v < G::kBPer; ++v) {
    const int s = tid + NTHR * v, row = s / CPR, c = (s % CPR) ^ swz_bits<CPR>(row);
    boff[v] = static_cast<uint32_t>(b_row(row)) * K + c * 16;
    bkc[v] = c * 16;
  }
  // K % BK may be any multiple of 16: the last stage's chunks past K read at
  // an offset past the buffer's end, which the hardware returns as zeros (an
  // exact zero term in every dot product)
  constexpr uint32_t kPastEnd = 0x80000000u;   // beyond any buffer resource here
  const uint32_t Ku = static_cast<uint32_t>(K);
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  auto issue = [&](int st) {
    uint8_t* base = w8_lds + (st % STAGES) * G::kStageBytes + wvu * kWave * 16;
    const uint32_t k0 = static_cast<uint32_t>(st) * BK;
#pragma unroll
    for (int v = 0; v < G::kAPer; ++v)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          a_rsrc, (lds_void_t*)(base + NTHR * v * 16), 16,
          k0 + akc[v] < Ku ? aoff[v] + k0 : kPastEnd, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < G::kBPer; ++v)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          b_rsrc, (lds_void_t*)(base + (G::kASlots + NTHR * v) * 16), 16,
          k0 + bkc[v] < Ku ? boff[v] + k0 : kPastEnd, 0, 0, 0);
  };

  // fixed size (see the slot arrays above); MI x NJ of it is used
  static_assert(MI <= 2 && NJ <= 4, "accumulator array holds 2 x 4 subtiles");
  i32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  const int steps = (K + BK - 1) / BK;
  // land the epilogue's kernel arguments now: a scalar load still in flight
  // inside the loop would turn every LDS wait there into a full drain
  asm volatile("" ::"s"(h_out), "s"(y_out), "s"(dbg_acc));
  // the stage's LDS reads, then its MFMAs
  auto compute = [&](const uint8_t* base) {
    i32x4_t aop[BK / 32][MI], bop[BK / 32][NJ];
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int c = 2 * ks + hf;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int arow = wm * RW + i * 32 + l32;
        aop[ks][i] = *reinterpret_cast<const i32x4_t*>(base + swz<CPR>(arow, c) * 16);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        bop[ks][j] = *reinterpret_cast<const i32x4_t*>(
            base + (G::kASlots + swz<CPR>(b_tile_row(j), c)) * 16);
    }
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks)
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop[ks][i], bop[ks][j], acc[i][j], 0, 0, 0);
    // keep that order through scheduling: later k-steps' reads land while the
    // first k-step's MFMAs run
    __builtin_amdgcn_sched_group_barrier(0x100, (BK / 32) * (MI + NJ), 0);
    __builtin_amdgcn_sched_group_barrier(0x008, (BK / 32) * MI * NJ, 0);
  };
  // An expert's last m-tile often holds only a few rows (at T 4096 about a
  // fifth of the tiles hold 32 rows or fewer): a wave whose row band lies past
  // the expert's rows takes no LDS reads and no MFMAs (its accumulators stay
  // zero and their stores are dropped); every other wave computes as usual.
  const bool band_live =
      __builtin_amdgcn_readfirstlane(wm) * RW < ti.p_end - ti.p_begin;   // uniform per wave

#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st)
    if (st < steps) issue(st);
  for (int st = 0; st < steps; ++st) {
    // stage st is complete once at most the later in-flight stages remain
    wait_stage<G::kLoadsPerStage, STAGES - 2>(min(STAGES - 2, steps - 1 - st));
    if (st + STAGES - 1 < steps) issue(st + STAGES - 1);
    if (band_live) compute(w8_lds + (st % STAGES) * G::kStageBytes);
  }

  // epilogue. C layout of a 32 x 32 subtile: lane holds column l32, rows
  // 8*(r/4) + 4*hf + (r%4).
  float cs[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) cs[j] = col_scale[b_tile_row(j)];
  const int mb = wm * RW + hf * 4;   // first tile row of this lane's C rows
  if (dbg_acc) {
    // the raw integer accumulators, for the tests (not the timed path)
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int p = ti.p_begin + mb + i * 32 + (r >> 2) * 8 + (r & 3);
        if (p >= ti.p_end) continue;
        int32_t* row = dbg_acc + static_cast<size_t>(p) * N;
        if (KIND == 0) {
#pragma unroll
          for (int j = 0; j < NJ / 2; ++j) {
            const int n = ti.nt * 128 + wn * HCW + j * 32 + l32;
            if (n >= I) continue;
            row[n] = acc[i][j][r];
            row[I + n] = acc[i][j + NJ / 2][r];
          }
        } else {
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const int n = ti.nt * kW8BN + wn * BW + j * 32 + l32;
            if (n < N) row[n] = acc[i][j][r];
          }
        }
      }
  }
  // Outputs go through a buffer resource based at the tile's first row and
  // column, one 4-byte store per element at a 32-bit offset: rows past the
  // expert's routed rows lie past the resource's end, and columns past the
  // row width are sent there too, so the hardware drops both (no branch and
  // no 64-bit address arithmetic per element).
  const int ow = (KIND == 0) ? I : N;                        // output row width
  const int cb = (KIND == 0) ? ti.nt * 128 : ti.nt * kW8BN;  // tile's first column
  const int rows = min(ti.p_end - ti.p_begin, BM);
  const uint32_t rowb = static_cast<uint32_t>(ow) * 4;
  float* obase = ((KIND == 0) ? h_out : y_out) + static_cast<size_t>(ti.p_begin) * ow + cb;
  const __amdgpu_buffer_rsrc_t o_rsrc =
      buffer_rsrc(obase, static_cast<uint32_t>(rows - 1) * rowb + static_cast<uint32_t>(ow - cb) * 4);
  constexpr int kOutCols = (KIND == 0) ? NJ / 2 : NJ;
  uint32_t coff[kOutCols];
#pragma unroll
  for (int j = 0; j < kOutCols; ++j) {
    const int c = (KIND == 0) ? (wn * HCW + j * 32 + l32) : (wn * BW + j * 32 + l32);
    coff[j] = cb + c < ow ? static_cast<uint32_t>(mb) * rowb + c * 4 : kPastEnd;
  }
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // the four consecutive rows 8q + 4hf + [0, 4) of subtile i
      const float4 rs4 = *reinterpret_cast<const float4*>(&row_scale[mb + i * 32 + q * 8]);
      const float rsv[4] = {rs4.x, rs4.y, rs4.z, rs4.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = q * 4 + t;
        const uint32_t roff = static_cast<uint32_t>(i * 32 + q * 8 + t) * rowb;
#pragma unroll
        for (int j = 0; j < kOutCols; ++j) {
          float v;
          if (KIND == 0) {
            const float g = static_cast<float>(acc[i][j][r]) * rsv[t] * cs[j];
            const float u = static_cast<float>(acc[i][j + NJ / 2][r]) * rsv[t] * cs[j + NJ / 2];
            v = silu_mul(g, u);
          } else {
            v = static_cast<float>(acc[i][j][r]) * rsv[t] * cs[j];
          }
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), o_rsrc,
                                                coff[j] + roff, 0, 0);
        }
      }
    }
  }
}

template <int KIND, class G>
hipError_t launch_w8a8_gemm(const int8_t* A, const float* a_scale, const int8_t* W,
                            const float* w_scale, const int* offsets, const int* sorted_slot,
                            int K, int N, int E, int topk, int T, float* h_out, float* y_out,
                            int32_t* dbg_acc, hipStream_t s) {
  const int NT = (KIND == 0) ? (N / 2 + 127) / 128 : (N + kW8BN - 1) / kW8BN;
  const long long R = static_cast<long long>(T) * topk;
  const long long act = R < E ? R : E;
  const long long mt_up = (R + G::BM - 1) / G::BM + act;
  long long grid = (mt_up * NT + 7) / 8 * 8;
  const size_t lds = static_cast<size_t>(G::kStages) * G::kStageBytes;
  const hipError_t e = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&w8a8_mfma_kernel<KIND, G>),
      hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((w8a8_mfma_kernel<KIND, G>), dim3(static_cast<unsigned>(grid)),
                     dim3(G::kThreads), lds, s, A, a_scale, W, w_scale, offsets, sorted_slot,
                     static_cast<int>(KIND == 0 ? T : R), K, N, E, topk, NT, h_out, y_out, dbg_acc);
  return hipGetLastError();
}

struct W8A8Ws {
  int8_t* xq;
  float* xs;
  float* h;
  int8_t* hq;
  float* hs;
};

W8A8Ws carve(void* ws, int T, int H, int I, int k) {
  const size_t R = static_cast<size_t>(T) * k;
  char* p = static_cast<char*>(ws);
  W8A8Ws w;
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

size_t w8a8_workspace_bytes(int T, int H, int I, int, int k) {
  const size_t R = static_cast<size_t>(T) * k;
  return align_up(static_cast<size_t>(T) * H, 256) + align_up(static_cast<size_t>(T) * 4, 256) +
         align_up(R * I * 4, 256) + align_up(R * I, 256) + align_up(R * 4, 256);
}

hipError_t launch_w8a8_ffn(int T, int H, int I, int E, int k, const uint16_t* x,
                           const int8_t* w13, const float* s13, const int8_t* w2,
                           const float* s2, const int* offsets, const int* sorted_slot,
                           const int*, const int*, float* y, const W8A8Debug& dbg, void* ws,
                           hipStream_t s) {
  if (T == 0) return hipSuccess;
  const W8A8Ws w = carve(ws, T, H, I, k);
  const int R = T * k;
  const int rows_per_block = kThreads / kWave;
  act_quant_kernel<<<(T + rows_per_block - 1) / rows_per_block, kThreads, 0, s>>>(
      x, T, H, w.xq, w.xs, dbg.xq, dbg.xs);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  err = launch_w8a8_gemm<0, W8Tile>(w.xq, w.xs, w13, s13, offsets, sorted_slot, H, 2 * I, E, k, T,
                                   w.h, nullptr, dbg.acc13, s);
  if (err != hipSuccess) return err;
  h_quant_kernel<<<(R + rows_per_block - 1) / rows_per_block, kThreads, 0, s>>>(
      w.h, R, I, w.hq, w.hs, dbg.hq, dbg.hs);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_w8a8_gemm<1, W8Tile>(w.hq, w.hs, w2, s2, offsets, sorted_slot, I, H, E, k, T,
                                    nullptr, y, dbg.acc2, s);
}

}  // namespace moe
