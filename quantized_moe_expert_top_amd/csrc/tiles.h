// Device-side tile lookup of the grouped GEMM kernels.
#pragma once
#include "common.h"

namespace moe {

// Locate this block's (expert, m-tile, n-tile). Tiles are ordered expert by
// expert, n-tile major and m-tile minor, so m-tiles that share a weight strip
// are adjacent; each XCD (blockIdx % 8) takes a contiguous run of tiles, so
// those neighbours share that XCD's L2. The expert's row range comes back
// through LDS with the tile (one round trip to memory in all); `sm_out` holds
// 5 ints.
struct TileInfo {
  int e, mt, nt, p_begin, p_end;
};

template <int BM, int NTHREADS = 256>
__device__ bool find_tile(const int* __restrict__ offsets, int E, int NT, int* sm_pref,
                          int* sm_out, TileInfo& ti) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid >> 6;
  const int ept = (E + NTHREADS - 1) / NTHREADS;  // <= 4
  int cnt[4], beg[4], rows_of[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * ept + i;
    int c = 0, b = 0, rows = 0;
    if (i < ept && e < E) {
      b = offsets[e];
      rows = offsets[e + 1] - b;
      c = (rows + BM - 1) / BM * NT;
    }
    beg[i] = b;
    rows_of[i] = rows;
    cnt[i] = c;
    sum += c;
  }
  int incl = sum;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += o;
  }
  if (lane == kWave - 1) sm_pref[wv] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < NTHREADS / kWave; ++i) {
    const int t = sm_pref[i];
    if (i < wv) before += t;
    total += t;
  }
  const int chunk = (total + 7) / 8;
  const int tau = (blockIdx.x & 7) * chunk + (blockIdx.x >> 3);
  const bool mine = (blockIdx.x >> 3) < chunk && tau < total;
  int start = before + incl - sum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (mine && tau >= start && tau < start + cnt[i]) {
      const int e = tid * ept + i;
      const int local = tau - start;
      const int mtiles = cnt[i] / NT;
      sm_out[0] = e;
      sm_out[1] = local % mtiles;
      sm_out[2] = local / mtiles;
      sm_out[3] = beg[i];
      sm_out[4] = beg[i] + rows_of[i];
    }
    start += cnt[i];
  }
  __syncthreads();
  if (!mine) return false;
  // the same for every thread of the block: kept in scalar registers, so
  // that buffer resources built from them need no per-lane handling
  ti.e = __builtin_amdgcn_readfirstlane(sm_out[0]);
  ti.mt = __builtin_amdgcn_readfirstlane(sm_out[1]);
  ti.nt = __builtin_amdgcn_readfirstlane(sm_out[2]);
  ti.p_begin = __builtin_amdgcn_readfirstlane(sm_out[3]) + ti.mt * BM;
  ti.p_end = __builtin_amdgcn_readfirstlane(sm_out[4]);
  return true;
}

}  // namespace moe
