// Host-side launchers of the libmoe kernels. Arguments have been validated by
// api.cpp before any of these runs; each returns the launch status.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr, int T, int H, int E,
                                float* logits, hipStream_t s);
hipError_t launch_route_topk(const float* logits, int T, int E, int k, int* ids, float* w,
                             hipStream_t s);

size_t permute_workspace_bytes(int T, int E, int k);
hipError_t launch_permute(const int* ids, int T, int E, int k, int* offsets, int* sorted_slot,
                          int* slot_pos, int* active, int* n_active, void* ws, hipStream_t s);

// W4A16: workspace holds h (bf16 [R, I]).
size_t w4a16_workspace_bytes(int T, int H, int I, int E, int k);
bool w4a16_uses_gemv(int T, int H, int I, int E, int k);
hipError_t launch_w4a16_ffn(int T, int H, int I, int E, int k, const uint16_t* x,
                            const uint8_t* w13, const uint16_t* s13, const uint8_t* w2,
                            const uint16_t* s2, const int* offsets, const int* sorted_slot,
                            const int* active, const int* n_active, float* y, void* ws,
                            hipStream_t s);

// Whole layer (route, permute, grouped FFN, combine); small T runs fused kernels.
size_t w4a16_layer_workspace_bytes(int T, int H, int I, int E, int k);
hipError_t launch_w4a16_layer(int T, int H, int I, int E, int k, const float* logits,
                              const uint16_t* x, const uint8_t* w13, const uint16_t* s13,
                              const uint8_t* w2, const uint16_t* s2, int* ids, float* w,
                              int* offsets, int* sorted_slot, int* slot_pos, int* active,
                              int* n_active, float* y, float* out, void* ws, hipStream_t s);

struct W8A8Debug {
  int8_t* xq;
  float* xs;
  int32_t* acc13;
  int8_t* hq;
  float* hs;
  int32_t* acc2;
};
size_t w8a8_workspace_bytes(int T, int H, int I, int E, int k);
hipError_t launch_w8a8_ffn(int T, int H, int I, int E, int k, const uint16_t* x,
                           const int8_t* w13, const float* s13, const int8_t* w2,
                           const float* s2, const int* offsets, const int* sorted_slot,
                           const int* active, const int* n_active, float* y,
                           const W8A8Debug& dbg, void* ws, hipStream_t s);

struct W4A8Debug {
  int8_t* xq;
  float* xs;
  int8_t* hq;
  float* hs;
};
size_t w4a8_workspace_bytes(int T, int H, int I, int E, int k);
hipError_t launch_w4a8_ffn(int T, int H, int I, int E, int k, const uint16_t* x,
                           const uint8_t* w13, const uint16_t* s13, const uint8_t* w2,
                           const uint16_t* s2, const int* offsets, const int* sorted_slot,
                           float* y, const W4A8Debug& dbg, void* ws, hipStream_t s);

hipError_t launch_expert_counts(const int* offsets, long long stride, int L, int E,
                                unsigned long long* counts, hipStream_t s);
hipError_t launch_hot_rank(const unsigned long long* counts, int L, int E, int n, int* hot,
                           hipStream_t s);
hipError_t launch_combine(const float* y, const int* slot_pos, const float* w, int T, int H,
                          int k, float* out, hipStream_t s);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace moe
