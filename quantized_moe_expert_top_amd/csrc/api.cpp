// libmoe C ABI: argument validation, device check, dispatch to the kernels.
// Every check runs on the host before anything is enqueued, so a non-OK
// status means no work was launched. Nothing here allocates or synchronizes.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/moe.h"
#include "launch.h"

namespace {

thread_local char g_last_error[512] = "";

moe_status fail(moe_status status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// 0 = unknown, 1 = gfx950, 2 = other arch
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

moe_status check_device() {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess)
    return fail(MOE_EDEVICE, "hipGetDevice: %s", hipGetErrorString(err));
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_EDEVICE, "device index %d out of range", dev);
  int state = g_arch_ok[dev].load(std::memory_order_acquire);
  if (state == 0) {
    hipDeviceProp_t prop;
    err = hipGetDeviceProperties(&prop, dev);
    if (err != hipSuccess)
      return fail(MOE_EDEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(err));
    state = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch_ok[dev].store(state, std::memory_order_release);
    if (state == 2)
      return fail(MOE_EUNSUPPORTED, "device %d is %s; libmoe runs on gfx950 only", dev,
                  prop.gcnArchName);
  }
  if (state == 2) return fail(MOE_EUNSUPPORTED, "device %d is not gfx950", dev);
  return MOE_OK;
}

moe_status launched(hipError_t err, const char* what) {
  if (err != hipSuccess) return fail(MOE_EDEVICE, "%s: %s", what, hipGetErrorString(err));
  return MOE_OK;
}

moe_status check_route_dims(int32_t T, int32_t E, int32_t k) {
  if (T < 0) return fail(MOE_EINVAL, "T = %d < 0", T);
  if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_ESHAPE, "E = %d outside [1, %d]", E, MOE_MAX_EXPERTS);
  if (k < 1 || k > E || k > MOE_MAX_TOPK)
    return fail(MOE_ESHAPE, "k = %d outside [1, min(E=%d, %d)]", k, E, MOE_MAX_TOPK);
  if (static_cast<long long>(T) * k >= (1LL << 31))
    return fail(MOE_ESHAPE, "T*k = %lld does not fit int32", static_cast<long long>(T) * k);
  return MOE_OK;
}

moe_status check_shape(const moe_shape* s, int hmod, int imod) {
  if (!s) return fail(MOE_EINVAL, "shape is NULL");
  moe_status st = check_route_dims(s->T, s->E, s->k);
  if (st) return st;
  if (s->H < hmod || s->H % hmod) return fail(MOE_ESHAPE, "H = %d must be a positive multiple of %d", s->H, hmod);
  if (s->I < imod || s->I % imod) return fail(MOE_ESHAPE, "I = %d must be a positive multiple of %d", s->I, imod);
  if (s->H > MOE_MAX_DIM || s->I > MOE_MAX_DIM)
    return fail(MOE_ESHAPE, "H = %d or I = %d above %d", s->H, s->I, MOE_MAX_DIM);
  const long long hi = s->H > s->I ? s->H : s->I;
  if (static_cast<long long>(s->T) * s->k * hi >= (1LL << 31))
    return fail(MOE_ESHAPE, "T*k*max(H, I) = %lld too large for 32-bit offsets",
                static_cast<long long>(s->T) * s->k * hi);
  if (2LL * s->H * s->I >= (1LL << 31))
    return fail(MOE_ESHAPE, "2*H*I = %lld too large for 32-bit offsets into one expert",
                2LL * s->H * s->I);
  return MOE_OK;
}

// Scratch of moe_layer_w4a16_noalloc: a file-scope device array, one copy per
// GPU, held until the process ends. In host code the array's name is only a
// host-side stand-in: its device address comes from hipGetSymbolAddress, taken
// once per device with that device current (on the entry point's first call
// there) and kept in g_scratch.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch[kMaxDevices];

moe_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return fail(MOE_EDEVICE, "hipGetDevice: %s", hipGetErrorString(err));
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_EDEVICE, "device index %d out of range", dev);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || p == nullptr)
      return fail(MOE_EDEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(err));
    g_scratch[dev].store(p, std::memory_order_release);   // racing threads store the same value
  }
  *out = p;
  return MOE_OK;
}

#define REQUIRE_PTR(p)                                              \
  do {                                                              \
    if (!(p)) return fail(MOE_EINVAL, "%s is NULL", #p);            \
    if (!aligned16(p)) return fail(MOE_EALIGN, "%s is not 16-byte aligned", #p); \
  } while (0)

}  // namespace

extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
    case MOE_ESHAPE: return "MOE_ESHAPE: unsupported shape";
    case MOE_EALIGN: return "MOE_EALIGN: pointer not 16-byte aligned";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace too small";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: device is not gfx950";
    case MOE_EDEVICE: return "MOE_EDEVICE: HIP runtime error";
    default: return "unknown moe_status";
  }
}

const char* moe_last_error(void) { return g_last_error; }

int moe_abi_version(void) { return MOE_ABI_VERSION; }

moe_status moe_router_logits(const uint16_t* x, const uint16_t* w_router, int32_t T, int32_t H,
                      int32_t E, float* logits, void* stream) {
  if (T < 0) return fail(MOE_EINVAL, "T = %d < 0", T);
  if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_ESHAPE, "E = %d outside [1, %d]", E, MOE_MAX_EXPERTS);
  if (H < 64 || H % 64) return fail(MOE_ESHAPE, "H = %d must be a positive multiple of 64", H);
  if (static_cast<long long>(T) * H >= (1LL << 31) || static_cast<long long>(E) * H >= (1LL << 31))
    return fail(MOE_ESHAPE, "T*H or E*H does not fit int32");
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(x);
  REQUIRE_PTR(w_router);
  REQUIRE_PTR(logits);
  moe_status st;
  if ((st = check_device()) != MOE_OK) return st;
  return launched(moe::launch_router_logits(x, w_router, T, H, E, logits,
                                            static_cast<hipStream_t>(stream)),
                  "moe_router_logits launch");
}

moe_status moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_ids,
                   float* topk_w, void* stream) {
  moe_status st = check_route_dims(T, E, k);
  if (st) return st;
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(logits);
  REQUIRE_PTR(topk_ids);
  REQUIRE_PTR(topk_w);
  if ((st = check_device()) != MOE_OK) return st;
  return launched(moe::launch_route_topk(logits, T, E, k, topk_ids, topk_w,
                                         static_cast<hipStream_t>(stream)),
                  "moe_route_topk launch");
}

size_t moe_permute_workspace(int32_t T, int32_t E, int32_t k) {
  if (check_route_dims(T, E, k)) return 0;
  return moe::permute_workspace_bytes(T, E, k);
}

moe_status moe_permute(const int32_t* topk_ids, int32_t T, int32_t E, int32_t k,
                int32_t* expert_offsets, int32_t* sorted_slot, int32_t* slot_pos,
                int32_t* active, int32_t* n_active, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_route_dims(T, E, k);
  if (st) return st;
  REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(n_active);
  if (T > 0) {
    REQUIRE_PTR(topk_ids);
    REQUIRE_PTR(sorted_slot);
    REQUIRE_PTR(slot_pos);
    REQUIRE_PTR(active);
  }
  const size_t need = moe::permute_workspace_bytes(T, E, k);
  if (need > 0) {
    if (ws_bytes < need)
      return fail(MOE_EWORKSPACE, "permute workspace %zu < %zu bytes", ws_bytes, need);
    REQUIRE_PTR(ws);
  }
  if ((st = check_device()) != MOE_OK) return st;
  return launched(moe::launch_permute(topk_ids, T, E, k, expert_offsets, sorted_slot, slot_pos,
                                      active, n_active, ws, static_cast<hipStream_t>(stream)),
                  "moe_permute launch");
}

size_t moe_w4a16_workspace(const moe_shape* s) {
  if (check_shape(s, MOE_GROUP, MOE_GROUP)) return 0;
  return moe::w4a16_workspace_bytes(s->T, s->H, s->I, s->E, s->k);
}

moe_status moe_grouped_w4a16_ffn(const moe_shape* s, const uint16_t* x, const uint8_t* w13,
                          const uint16_t* s13, const uint8_t* w2, const uint16_t* s2,
                          const int32_t* expert_offsets, const int32_t* sorted_slot,
                          const int32_t* active, const int32_t* n_active, float* y, void* ws,
                          size_t ws_bytes, void* stream) {
  moe_status st = check_shape(s, MOE_GROUP, MOE_GROUP);
  if (st) return st;
  if (s->T == 0) return MOE_OK;
  REQUIRE_PTR(x);
  REQUIRE_PTR(w13);
  REQUIRE_PTR(s13);
  REQUIRE_PTR(w2);
  REQUIRE_PTR(s2);
  REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(sorted_slot);
  REQUIRE_PTR(active);
  REQUIRE_PTR(n_active);
  REQUIRE_PTR(y);
  const size_t need = moe::w4a16_workspace_bytes(s->T, s->H, s->I, s->E, s->k);
  if (ws_bytes < need) return fail(MOE_EWORKSPACE, "w4a16 workspace %zu < %zu bytes", ws_bytes, need);
  REQUIRE_PTR(ws);
  if ((st = check_device()) != MOE_OK) return st;
  return launched(moe::launch_w4a16_ffn(s->T, s->H, s->I, s->E, s->k, x, w13, s13, w2, s2,
                                        expert_offsets, sorted_slot, active, n_active, y, ws,
                                        static_cast<hipStream_t>(stream)),
                  "moe_grouped_w4a16_ffn launch");
}

size_t moe_layer_w4a16_workspace(const moe_shape* s) {
  if (check_shape(s, MOE_GROUP, MOE_GROUP)) return 0;
  return moe::w4a16_layer_workspace_bytes(s->T, s->H, s->I, s->E, s->k);
}

moe_status moe_layer_w4a16(const moe_shape* s, const float* logits, const uint16_t* x,
                    const uint8_t* w13, const uint16_t* s13, const uint8_t* w2,
                    const uint16_t* s2, int32_t* topk_ids, float* topk_w,
                    int32_t* expert_offsets, int32_t* sorted_slot, int32_t* slot_pos,
                    int32_t* active, int32_t* n_active, float* y, float* out, void* ws,
                    size_t ws_bytes, void* stream) {
  moe_status st = check_shape(s, MOE_GROUP, MOE_GROUP);
  if (st) return st;
  REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(n_active);
  const size_t need = moe::w4a16_layer_workspace_bytes(s->T, s->H, s->I, s->E, s->k);
  if (ws_bytes < need) return fail(MOE_EWORKSPACE, "layer workspace %zu < %zu bytes", ws_bytes, need);
  REQUIRE_PTR(ws);
  if (s->T > 0) {
    REQUIRE_PTR(logits);
    REQUIRE_PTR(x);
    REQUIRE_PTR(w13);
    REQUIRE_PTR(s13);
    REQUIRE_PTR(w2);
    REQUIRE_PTR(s2);
    REQUIRE_PTR(topk_ids);
    REQUIRE_PTR(topk_w);
    REQUIRE_PTR(sorted_slot);
    REQUIRE_PTR(slot_pos);
    REQUIRE_PTR(active);
    REQUIRE_PTR(y);
    REQUIRE_PTR(out);
  }
  if ((st = check_device()) != MOE_OK) return st;
  return launched(moe::launch_w4a16_layer(s->T, s->H, s->I, s->E, s->k, logits, x, w13, s13, w2,
                                          s2, topk_ids, topk_w, expert_offsets, sorted_slot,
                                          slot_pos, active, n_active, y, out, ws,
                                          static_cast<hipStream_t>(stream)),
                  "moe_layer_w4a16 launch");
}

moe_status moe_layer_w4a16_noalloc(const moe_shape* s, const float* logits, const uint16_t* x,
                                   const uint8_t* w13, const uint16_t* s13, const uint8_t* w2,
                                   const uint16_t* s2, int32_t* topk_ids, float* topk_w,
                                   int32_t* expert_offsets, int32_t* sorted_slot,
                                   int32_t* slot_pos, int32_t* active, int32_t* n_active,
                                   float* y, float* out, void* stream) {
  moe_status st = check_shape(s, MOE_GROUP, MOE_GROUP);
  if (st) return st;
  const size_t need = moe::w4a16_layer_workspace_bytes(s->T, s->H, s->I, s->E, s->k);
  if (need > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_EWORKSPACE,
                "this shape needs %zu bytes of scratch; the static scratch of "
                "moe_layer_w4a16_noalloc holds %zu (use moe_layer_w4a16 with a workspace)",
                need, static_cast<size_t>(MOE_NOALLOC_SCRATCH_BYTES));
  REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(n_active);
  if (s->T > 0) {
    REQUIRE_PTR(logits);
    REQUIRE_PTR(x);
    REQUIRE_PTR(w13);
    REQUIRE_PTR(s13);
    REQUIRE_PTR(w2);
    REQUIRE_PTR(s2);
    REQUIRE_PTR(topk_ids);
    REQUIRE_PTR(topk_w);
    REQUIRE_PTR(sorted_slot);
    REQUIRE_PTR(slot_pos);
    REQUIRE_PTR(active);
    REQUIRE_PTR(y);
    REQUIRE_PTR(out);
  }
  if ((st = check_device()) != MOE_OK) return st;
  void* ws = nullptr;
  if ((st = scratch_of_current_device(&ws)) != MOE_OK) return st;
  return launched(moe::launch_w4a16_layer(s->T, s->H, s->I, s->E, s->k, logits, x, w13, s13, w2,
                                          s2, topk_ids, topk_w, expert_offsets, sorted_slot,
                                          slot_pos, active, n_active, y, out, ws,
                                          static_cast<hipStream_t>(stream)),
                  "moe_layer_w4a16_noalloc launch");
}

size_t moe_w4a8_workspace(const moe_shape* s) {
  if (check_shape(s, MOE_GROUP, MOE_GROUP)) return 0;
  return moe::w4a8_workspace_bytes(s->T, s->H, s->I, s->E, s->k);
}

moe_status moe_grouped_w4a8_ffn(const moe_shape* s, const uint16_t* x, const uint8_t* w13,
                         const uint16_t* s13, const uint8_t* w2, const uint16_t* s2,
                         const int32_t* expert_offsets, const int32_t* sorted_slot,
                         const int32_t* active, const int32_t* n_active, float* y,
                         const moe_w4a8_debug* dbg, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_shape(s, MOE_GROUP, MOE_GROUP);
  if (st) return st;
  if (s->T == 0) return MOE_OK;
  REQUIRE_PTR(x);
  REQUIRE_PTR(w13);
  REQUIRE_PTR(s13);
  REQUIRE_PTR(w2);
  REQUIRE_PTR(s2);
  REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(sorted_slot);
  REQUIRE_PTR(active);
  REQUIRE_PTR(n_active);
  REQUIRE_PTR(y);
  moe::W4A8Debug d = {nullptr, nullptr, nullptr, nullptr};
  if (dbg) {
    d = {dbg->xq, dbg->xs, dbg->hq, dbg->hs};
    const void* ps[4] = {d.xq, d.xs, d.hq, d.hs};
    for (const void* p : ps)
      if (p && !aligned16(p)) return fail(MOE_EALIGN, "a debug pointer is not 16-byte aligned");
  }
  const size_t need = moe::w4a8_workspace_bytes(s->T, s->H, s->I, s->E, s->k);
  if (ws_bytes < need) return fail(MOE_EWORKSPACE, "w4a8 workspace %zu < %zu bytes", ws_bytes, need);
  REQUIRE_PTR(ws);
  if ((st = check_device()) != MOE_OK) return st;
  return launched(moe::launch_w4a8_ffn(s->T, s->H, s->I, s->E, s->k, x, w13, s13, w2, s2,
                                       expert_offsets, sorted_slot, y, d, ws,
                                       static_cast<hipStream_t>(stream)),
                  "moe_grouped_w4a8_ffn launch");
}

size_t moe_w8a8_workspace(const moe_shape* s) {
  if (check_shape(s, 16, 16)) return 0;
  return moe::w8a8_workspace_bytes(s->T, s->H, s->I, s->E, s->k);
}

moe_status moe_grouped_w8a8_ffn(const moe_shape* s, const uint16_t* x, const int8_t* w13,
                         const float* s13, const int8_t* w2, const float* s2,
                         const int32_t* expert_offsets, const int32_t* sorted_slot,
                         const int32_t* active, const int32_t* n_active, float* y,
                         const moe_w8a8_debug* dbg, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_shape(s, 16, 16);
  if (st) return st;
  if (s->T == 0) return MOE_OK;
  REQUIRE_PTR(x);
  REQUIRE_PTR(w13);
  REQUIRE_PTR(s13);
  REQUIRE_PTR(w2);
  REQUIRE_PTR(s2);
  REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(sorted_slot);
  REQUIRE_PTR(active);
  REQUIRE_PTR(n_active);
  REQUIRE_PTR(y);
  moe::W8A8Debug d = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  if (dbg) {
    d = {dbg->xq, dbg->xs, dbg->acc13, dbg->hq, dbg->hs, dbg->acc2};
    const void* ps[6] = {d.xq, d.xs, d.acc13, d.hq, d.hs, d.acc2};
    for (const void* p : ps)
      if (p && !aligned16(p)) return fail(MOE_EALIGN, "a debug pointer is not 16-byte aligned");
  }
  const size_t need = moe::w8a8_workspace_bytes(s->T, s->H, s->I, s->E, s->k);
  if (ws_bytes < need) return fail(MOE_EWORKSPACE, "w8a8 workspace %zu < %zu bytes", ws_bytes, need);
  REQUIRE_PTR(ws);
  if ((st = check_device()) != MOE_OK) return st;
  return launched(moe::launch_w8a8_ffn(s->T, s->H, s->I, s->E, s->k, x, w13, s13, w2, s2,
                                       expert_offsets, sorted_slot, active, n_active, y, d, ws,
                                       static_cast<hipStream_t>(stream)),
                  "moe_grouped_w8a8_ffn launch");
}

moe_status moe_combine(const float* y, const int32_t* slot_pos, const float* topk_w, int32_t T,
                int32_t H, int32_t k, float* out, void* stream) {
  if (T < 0) return fail(MOE_EINVAL, "T = %d < 0", T);
  if (k < 1 || k > MOE_MAX_TOPK) return fail(MOE_ESHAPE, "k = %d outside [1, %d]", k, MOE_MAX_TOPK);
  if (H < 8 || H % 8) return fail(MOE_ESHAPE, "H = %d must be a positive multiple of 8", H);
  if (static_cast<long long>(T) * k * H >= (1LL << 31))
    return fail(MOE_ESHAPE, "T*k*H too large for int32 row indexing");
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(y);
  REQUIRE_PTR(slot_pos);
  REQUIRE_PTR(topk_w);
  REQUIRE_PTR(out);
  moe_status st = check_device();
  if (st) return st;
  return launched(moe::launch_combine(y, slot_pos, topk_w, T, H, k, out,
                                      static_cast<hipStream_t>(stream)),
                  "moe_combine launch");
}

moe_status moe_expert_counts_accumulate(const int32_t* expert_offsets, int64_t offsets_stride,
                                 int32_t L, int32_t E, uint64_t* counts, void* stream) {
  if (L < 0) return fail(MOE_EINVAL, "L = %d < 0", L);
  if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_ESHAPE, "E = %d outside [1, %d]", E, MOE_MAX_EXPERTS);
  if (offsets_stride < static_cast<int64_t>(E) + 1)
    return fail(MOE_ESHAPE, "offsets_stride = %lld < E + 1", static_cast<long long>(offsets_stride));
  if (L == 0) return MOE_OK;
  REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(counts);
  moe_status st;
  if ((st = check_device()) != MOE_OK) return st;
  return launched(moe::launch_expert_counts(expert_offsets, offsets_stride, L, E,
                                            reinterpret_cast<unsigned long long*>(counts),
                                            static_cast<hipStream_t>(stream)),
                  "moe_expert_counts_accumulate launch");
}

moe_status moe_expert_hot_rank(const uint64_t* counts, int32_t L, int32_t E, int32_t n, int32_t* hot_ids,
                        void* stream) {
  if (L < 0) return fail(MOE_EINVAL, "L = %d < 0", L);
  if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_ESHAPE, "E = %d outside [1, %d]", E, MOE_MAX_EXPERTS);
  if (n < 0 || n > E) return fail(MOE_ESHAPE, "n = %d outside [0, E = %d]", n, E);
  if (L == 0 || n == 0) return MOE_OK;
  REQUIRE_PTR(counts);
  REQUIRE_PTR(hot_ids);
  moe_status st;
  if ((st = check_device()) != MOE_OK) return st;
  return launched(moe::launch_hot_rank(reinterpret_cast<const unsigned long long*>(counts), L, E, n,
                                       hot_ids, static_cast<hipStream_t>(stream)),
                  "moe_expert_hot_rank launch");
}

}  // extern "C"
