"""ctypes binding of libmoe (argument marshalling only).

Every function takes torch tensors that already live on the GPU, passes their
device pointers and the current HIP stream to the C ABI, and raises MoeError on
a non-OK status. All arithmetic happens in libmoe's HIP kernels; there is no
fallback: if libmoe.so is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

STATUS = {0: "MOE_OK", 1: "MOE_EINVAL", 2: "MOE_ESHAPE", 3: "MOE_EALIGN",
          4: "MOE_EWORKSPACE", 5: "MOE_EUNSUPPORTED", 6: "MOE_EDEVICE"}

EXPORTS = ("moe_status_str", "moe_last_error", "moe_abi_version", "moe_router_logits",
           "moe_route_topk",
           "moe_permute_workspace", "moe_permute", "moe_w4a16_workspace",
           "moe_grouped_w4a16_ffn", "moe_w4a8_workspace", "moe_grouped_w4a8_ffn",
           "moe_w8a8_workspace", "moe_grouped_w8a8_ffn", "moe_expert_counts_accumulate",
           "moe_expert_hot_rank",
           "moe_combine", "moe_layer_w4a16_workspace", "moe_layer_w4a16",
           "moe_layer_w4a16_noalloc")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        self.status = status
        super().__init__(f"{fn} -> {STATUS.get(status, status)}: {detail}")


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32)]


class MoeW8A8Debug(ctypes.Structure):
    _fields_ = [("xq", ctypes.c_void_p), ("xs", ctypes.c_void_p), ("acc13", ctypes.c_void_p),
                ("hq", ctypes.c_void_p), ("hs", ctypes.c_void_p), ("acc2", ctypes.c_void_p)]


class MoeW4A8Debug(ctypes.Structure):
    _fields_ = [("xq", ctypes.c_void_p), ("xs", ctypes.c_void_p), ("hq", ctypes.c_void_p),
                ("hs", ctypes.c_void_p)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoe.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libmoe.so not built at {path}; run __graft_entry__.build() or "
                           "python -m quantized_moe_expert_top_amd.build")
    # libmoe must bind to the HIP runtime that owns the process's device memory
    # and streams. torch ships its own libamdhip64 (same soname as ROCm's), so
    # import it first: the dynamic loader then reuses that copy instead of
    # mapping a second HIP/HSA runtime from ROCm's directory.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise RuntimeError(f"two HIP runtimes mapped in this process: {runtimes}")
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "moe_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_abi_version": (ctypes.c_int, []),
        "moe_router_logits": (ctypes.c_int, [P, P, I32, I32, I32, P, P]),
        "moe_expert_counts_accumulate": (ctypes.c_int, [P, ctypes.c_int64, I32, I32, P, P]),
        "moe_expert_hot_rank": (ctypes.c_int, [P, I32, I32, I32, P, P]),
        "moe_route_topk": (ctypes.c_int, [P, I32, I32, I32, P, P, P]),
        "moe_permute_workspace": (SZ, [I32, I32, I32]),
        "moe_permute": (ctypes.c_int, [P, I32, I32, I32, P, P, P, P, P, P, SZ, P]),
        "moe_w4a16_workspace": (SZ, [ctypes.POINTER(MoeShape)]),
        "moe_grouped_w4a16_ffn": (ctypes.c_int, [ctypes.POINTER(MoeShape)] + [P] * 11 + [SZ, P]),
        "moe_w4a8_workspace": (SZ, [ctypes.POINTER(MoeShape)]),
        "moe_grouped_w4a8_ffn": (ctypes.c_int, [ctypes.POINTER(MoeShape)] + [P] * 10 +
                                 [ctypes.POINTER(MoeW4A8Debug), P, SZ, P]),
        "moe_w8a8_workspace": (SZ, [ctypes.POINTER(MoeShape)]),
        "moe_grouped_w8a8_ffn": (ctypes.c_int, [ctypes.POINTER(MoeShape)] + [P] * 10 +
                                 [ctypes.POINTER(MoeW8A8Debug), P, SZ, P]),
        "moe_combine": (ctypes.c_int, [P, P, P, I32, I32, I32, P, P]),
        "moe_layer_w4a16_workspace": (SZ, [ctypes.POINTER(MoeShape)]),
        "moe_layer_w4a16": (ctypes.c_int, [ctypes.POINTER(MoeShape)] + [P] * 16 + [SZ, P]),
        "moe_layer_w4a16_noalloc": (ctypes.c_int, [ctypes.POINTER(MoeShape)] + [P] * 16),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _hip_runtimes_mapped() -> list:
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


def _check(fn: str, status: int) -> None:
    if status != 0:
        detail = load().moe_last_error().decode(errors="replace")
        raise MoeError(fn, status, detail)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _need(t, nbytes: int, name: str) -> None:
    """Host-side size check: the C ABI receives bare pointers, so make sure each
    tensor covers the bytes the kernels will touch before launching."""
    if t is None:
        return
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name} holds {have} bytes, the call needs {nbytes}")


def _stream(stream) -> int | None:
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ------------------------------------------------------------- raw calls ----
def router_logits(x, w_router, logits, stream=None) -> None:
    T, H = x.shape
    E = w_router.shape[0]
    _need(x, T * H * 2, "x")
    _need(w_router, E * H * 2, "w_router")
    _need(logits, T * E * 4, "logits")
    _check("moe_router_logits", load().moe_router_logits(_ptr(x), _ptr(w_router), T, H, E,
                                                         _ptr(logits), _stream(stream)))


def expert_counts_accumulate(expert_offsets, counts, stream=None) -> None:
    """counts [L, E] uint64 (int64 tensor) += per-expert rows of each layer's
    expert_offsets [L, stride >= E + 1] (or [E + 1] with counts [E])."""
    L, E = (1, counts.shape[0]) if counts.dim() == 1 else tuple(counts.shape)
    stride = expert_offsets.shape[-1] if expert_offsets.dim() > 1 else E + 1
    if L > 0:
        _need(expert_offsets, ((L - 1) * stride + E + 1) * 4, "expert_offsets")
        _need(counts, L * E * 8, "counts")
    _check("moe_expert_counts_accumulate", load().moe_expert_counts_accumulate(
        _ptr(expert_offsets), stride, L, E, _ptr(counts), _stream(stream)))


def expert_hot_rank(counts, n: int, hot_ids, stream=None) -> None:
    """hot_ids [L, n] int32 = each layer's n most-loaded experts (descending,
    ties to the lower index) from counts [L, E] (or [E] with hot_ids [n])."""
    L, E = (1, counts.shape[0]) if counts.dim() == 1 else tuple(counts.shape)
    if L > 0 and n > 0:
        _need(counts, L * E * 8, "counts")
        _need(hot_ids, L * n * 4, "hot_ids")
    _check("moe_expert_hot_rank", load().moe_expert_hot_rank(_ptr(counts), L, E, n, _ptr(hot_ids),
                                                             _stream(stream)))


def route_topk(logits, k: int, topk_ids, topk_w, stream=None) -> None:
    T, E = logits.shape
    _need(logits, T * E * 4, "logits")
    _need(topk_ids, T * k * 4, "topk_ids")
    _need(topk_w, T * k * 4, "topk_w")
    _check("moe_route_topk", load().moe_route_topk(_ptr(logits), T, E, k, _ptr(topk_ids),
                                                   _ptr(topk_w), _stream(stream)))


def permute_workspace(T: int, E: int, k: int) -> int:
    return int(load().moe_permute_workspace(T, E, k))


def permute(topk_ids, E: int, expert_offsets, sorted_slot, slot_pos, active, n_active,
            ws=None, stream=None) -> None:
    T, k = topk_ids.shape
    R = T * k
    _need(topk_ids, R * 4, "topk_ids")
    _need(expert_offsets, (E + 1) * 4, "expert_offsets")
    _need(sorted_slot, R * 4, "sorted_slot")
    _need(slot_pos, R * 4, "slot_pos")
    _need(active, min(E, R) * 4, "active")
    _need(n_active, 4, "n_active")
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("moe_permute", load().moe_permute(_ptr(topk_ids), T, E, k, _ptr(expert_offsets),
                                             _ptr(sorted_slot), _ptr(slot_pos), _ptr(active),
                                             _ptr(n_active), _ptr(ws), nbytes, _stream(stream)))


def w4a16_workspace(T: int, H: int, I: int, E: int, k: int) -> int:
    s = MoeShape(T, H, I, E, k)
    return int(load().moe_w4a16_workspace(ctypes.byref(s)))


def _check_ffn_sizes(shape, x, expert_offsets, sorted_slot, active, n_active, y):
    T, H, I, E, k = shape
    R = T * k
    _need(x, T * H * 2, "x")
    _need(expert_offsets, (E + 1) * 4, "expert_offsets")
    _need(sorted_slot, R * 4, "sorted_slot")
    _need(active, min(E, R) * 4, "active")
    _need(n_active, 4, "n_active")
    _need(y, R * H * 4, "y")


def grouped_w4a16_ffn(shape, x, w13, s13, w2, s2, expert_offsets, sorted_slot, active,
                      n_active, y, ws, stream=None) -> None:
    T, H, I, E, k = shape
    if T > 0 and H % 128 == 0 and I % 128 == 0:
        _check_ffn_sizes(shape, x, expert_offsets, sorted_slot, active, n_active, y)
        _need(w13, E * 2 * I * H // 2, "w13")
        _need(s13, E * 2 * I * (H // 128) * 2, "s13")
        _need(w2, E * H * I // 2, "w2")
        _need(s2, E * H * (I // 128) * 2, "s2")
    s = MoeShape(*shape)
    nbytes = ws.numel() * ws.element_size()
    _check("moe_grouped_w4a16_ffn", load().moe_grouped_w4a16_ffn(
        ctypes.byref(s), _ptr(x), _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2),
        _ptr(expert_offsets), _ptr(sorted_slot), _ptr(active), _ptr(n_active), _ptr(y),
        _ptr(ws), nbytes, _stream(stream)))


def w4a8_workspace(T: int, H: int, I: int, E: int, k: int) -> int:
    s = MoeShape(T, H, I, E, k)
    return int(load().moe_w4a8_workspace(ctypes.byref(s)))


def grouped_w4a8_ffn(shape, x, w13, s13, w2, s2, expert_offsets, sorted_slot, active,
                     n_active, y, ws, debug: dict | None = None, stream=None) -> None:
    T, H, I, E, k = shape
    R = T * k
    if T > 0 and H % 128 == 0 and I % 128 == 0:
        _check_ffn_sizes(shape, x, expert_offsets, sorted_slot, active, n_active, y)
        _need(w13, E * 2 * I * H // 2, "w13")
        _need(s13, E * 2 * I * (H // 128) * 2, "s13")
        _need(w2, E * H * I // 2, "w2")
        _need(s2, E * H * (I // 128) * 2, "s2")
        if debug:
            for n, nb in (("xq", T * H), ("xs", T * 4), ("hq", R * I), ("hs", R * 4)):
                _need(debug.get(n), nb, "debug." + n)
    s = MoeShape(*shape)
    dbg = None
    if debug:
        dbg = ctypes.byref(MoeW4A8Debug(*[_ptr(debug.get(n)) for n in ("xq", "xs", "hq", "hs")]))
    nbytes = ws.numel() * ws.element_size()
    _check("moe_grouped_w4a8_ffn", load().moe_grouped_w4a8_ffn(
        ctypes.byref(s), _ptr(x), _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2),
        _ptr(expert_offsets), _ptr(sorted_slot), _ptr(active), _ptr(n_active), _ptr(y),
        dbg, _ptr(ws), nbytes, _stream(stream)))


def w8a8_workspace(T: int, H: int, I: int, E: int, k: int) -> int:
    s = MoeShape(T, H, I, E, k)
    return int(load().moe_w8a8_workspace(ctypes.byref(s)))


def grouped_w8a8_ffn(shape, x, w13, s13, w2, s2, expert_offsets, sorted_slot, active,
                     n_active, y, ws, debug: dict | None = None, stream=None) -> None:
    T, H, I, E, k = shape
    R = T * k
    if T > 0 and H % 16 == 0 and I % 16 == 0:
        _check_ffn_sizes(shape, x, expert_offsets, sorted_slot, active, n_active, y)
        _need(w13, E * 2 * I * H, "w13")
        _need(s13, E * 2 * I * 4, "s13")
        _need(w2, E * H * I, "w2")
        _need(s2, E * H * 4, "s2")
        if debug:
            for n, nb in (("xq", T * H), ("xs", T * 4), ("acc13", R * 2 * I * 4),
                          ("hq", R * I), ("hs", R * 4), ("acc2", R * H * 4)):
                _need(debug.get(n), nb, "debug." + n)
    s = MoeShape(*shape)
    dbg = None
    if debug:
        dbg = ctypes.byref(MoeW8A8Debug(*[_ptr(debug.get(n)) for n in
                                          ("xq", "xs", "acc13", "hq", "hs", "acc2")]))
    nbytes = ws.numel() * ws.element_size()
    _check("moe_grouped_w8a8_ffn", load().moe_grouped_w8a8_ffn(
        ctypes.byref(s), _ptr(x), _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2),
        _ptr(expert_offsets), _ptr(sorted_slot), _ptr(active), _ptr(n_active), _ptr(y),
        dbg, _ptr(ws), nbytes, _stream(stream)))


def combine(y, slot_pos, topk_w, out, stream=None) -> None:
    T, k = topk_w.shape
    H = y.shape[1]
    _need(y, T * k * H * 4, "y")
    _need(slot_pos, T * k * 4, "slot_pos")
    _need(topk_w, T * k * 4, "topk_w")
    _need(out, T * H * 4, "out")
    _check("moe_combine", load().moe_combine(_ptr(y), _ptr(slot_pos), _ptr(topk_w), T, H, k,
                                             _ptr(out), _stream(stream)))


def layer_w4a16_workspace(T: int, H: int, I: int, E: int, k: int) -> int:
    s = MoeShape(T, H, I, E, k)
    return int(load().moe_layer_w4a16_workspace(ctypes.byref(s)))


def _check_layer_sizes(shape, logits, x, w13, s13, w2, s2, topk_ids, topk_w, expert_offsets,
                       sorted_slot, slot_pos, active, n_active, y, out) -> None:
    T, H, I, E, k = shape
    R = T * k
    if T > 0 and H % 128 == 0 and I % 128 == 0:
        _check_ffn_sizes(shape, x, expert_offsets, sorted_slot, active, n_active, y)
        _need(logits, T * E * 4, "logits")
        _need(w13, E * 2 * I * H // 2, "w13")
        _need(s13, E * 2 * I * (H // 128) * 2, "s13")
        _need(w2, E * H * I // 2, "w2")
        _need(s2, E * H * (I // 128) * 2, "s2")
        _need(topk_ids, R * 4, "topk_ids")
        _need(topk_w, R * 4, "topk_w")
        _need(slot_pos, R * 4, "slot_pos")
        _need(out, T * H * 4, "out")


def layer_w4a16_noalloc(shape, logits, x, w13, s13, w2, s2, topk_ids, topk_w, expert_offsets,
                        sorted_slot, slot_pos, active, n_active, y, out, stream=None) -> None:
    """moe_layer_w4a16 on the library's static scratch (no workspace argument)."""
    _check_layer_sizes(shape, logits, x, w13, s13, w2, s2, topk_ids, topk_w, expert_offsets,
                       sorted_slot, slot_pos, active, n_active, y, out)
    s = MoeShape(*shape)
    _check("moe_layer_w4a16_noalloc", load().moe_layer_w4a16_noalloc(
        ctypes.byref(s), _ptr(logits), _ptr(x), _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2),
        _ptr(topk_ids), _ptr(topk_w), _ptr(expert_offsets), _ptr(sorted_slot), _ptr(slot_pos),
        _ptr(active), _ptr(n_active), _ptr(y), _ptr(out), _stream(stream)))


def layer_w4a16(shape, logits, x, w13, s13, w2, s2, topk_ids, topk_w, expert_offsets,
                sorted_slot, slot_pos, active, n_active, y, out, ws, stream=None) -> None:
    _check_layer_sizes(shape, logits, x, w13, s13, w2, s2, topk_ids, topk_w, expert_offsets,
                       sorted_slot, slot_pos, active, n_active, y, out)
    s = MoeShape(*shape)
    nbytes = ws.numel() * ws.element_size()
    _check("moe_layer_w4a16", load().moe_layer_w4a16(
        ctypes.byref(s), _ptr(logits), _ptr(x), _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2),
        _ptr(topk_ids), _ptr(topk_w), _ptr(expert_offsets), _ptr(sorted_slot), _ptr(slot_pos),
        _ptr(active), _ptr(n_active), _ptr(y), _ptr(out), _ptr(ws), nbytes, _stream(stream)))
