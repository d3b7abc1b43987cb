"""Host-only checks of libmoe's C ABI: the library loads, exports every symbol
include/moe.h declares, and every validation error is reachable before any
device work (no kernels run here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

try:
    from quantized_moe_expert_top_amd import _lib
    LIB = _lib.load()
except RuntimeError as exc:  # not built
    LIB = None
    REASON = str(exc)

needs_lib = pytest.mark.skipif(LIB is None, reason="libmoe.so not built")

A = 0x10000          # a 16-byte aligned stand-in address, never dereferenced on the host
B = 0x20000
MIS = 0x10004        # misaligned


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text)))


@needs_lib
def test_exports_match_header():
    names = header_functions()
    assert len(names) == 19
    for n in names:
        assert hasattr(LIB, n), n
    assert set(names) == set(_lib.EXPORTS)


@needs_lib
def test_version_and_status_strings():
    assert LIB.moe_abi_version() == 1
    for s in range(7):
        assert LIB.moe_status_str(s).decode().startswith(_lib.STATUS[s])
    assert b"unknown" in LIB.moe_status_str(99)


def _no_gpu():
    try:
        import torch
        return not torch.cuda.is_available()
    except Exception:
        return True


@needs_lib
@pytest.mark.parametrize("args,status", [
    ((A, 4, 8, 2, A, B), 6 if _no_gpu() else None),   # valid -> device check
    ((MIS, 4, 8, 2, A, B), 3),
    ((None, 4, 8, 2, A, B), 1),
    ((A, 4, 8, 0, A, B), 2),
    ((A, 4, 8, 9, A, B), 2),
    ((A, 4, 0, 1, A, B), 2),
    ((A, 4, 1025, 2, A, B), 2),
    ((A, 4, 64, 33, A, B), 2),
    ((A, -1, 8, 2, A, B), 1),
    ((A, 0, 8, 2, None, None), 0),                      # empty batch is a no-op
])
def test_route_validation(args, status):
    if status is None:
        pytest.skip("a GPU is present; the valid call would launch")
    assert LIB.moe_route_topk(*args, None) == status
    if status:
        assert LIB.moe_last_error()


@needs_lib
def test_permute_validation_and_workspace():
    assert _lib.permute_workspace(2, 128, 8) == 0              # single block
    ws = _lib.permute_workspace(4096, 128, 8)
    assert ws == 2 * 32 * 128 * 4
    f = LIB.moe_permute
    # workspace too small for the multi-block path
    assert f(A, 4096, 128, 8, A, A, A, A, A, A, ws - 4, None) == 4
    assert f(A, 4096, 128, 8, A, A, A, A, A, None, ws, None) == 1
    assert f(A, 4, 8, 2, None, A, A, A, A, None, 0, None) == 1
    assert f(A, 4, 8, 2, A, A, MIS, A, A, None, 0, None) == 3
    assert f(A, 4, 8, 9, A, A, A, A, A, None, 0, None) == 2
    if _no_gpu():
        assert f(A, 4, 8, 2, A, A, A, A, A, None, 0, None) == 6
        assert f(None, 0, 8, 2, A, None, None, None, A, None, 0, None) == 6   # T=0 still writes offsets


def _shape(T=4, H=256, I=128, E=8, k=2):
    return _lib.MoeShape(T, H, I, E, k)


@needs_lib
def test_w4a16_validation():
    f = LIB.moe_grouped_w4a16_ffn
    s = _shape()
    need = _lib.w4a16_workspace(4, 256, 128, 8, 2)
    assert need == 4 * 2 * 128 * 2      # h: bf16 [T*k, I], already a multiple of 256 bytes
    ok = [A] * 10          # x, w13, s13, w2, s2, offsets, sorted_slot, active, n_active, y
    assert f(ctypes.byref(_shape(H=200)), *ok, A, need, None) == 2     # H % 128
    assert f(ctypes.byref(_shape(I=64)), *ok, A, need, None) == 2      # I % 128
    assert f(ctypes.byref(_shape(k=9)), *ok, A, need, None) == 2
    assert f(ctypes.byref(_shape(I=16512)), *ok, A, need, None) == 2        # I > MOE_MAX_DIM
    assert f(None, *ok, A, need, None) == 1
    assert f(ctypes.byref(s), *ok, A, need - 1, None) == 4
    bad = list(ok)
    bad[4] = MIS
    assert f(ctypes.byref(s), *bad, A, need, None) == 3
    bad[4] = None
    assert f(ctypes.byref(s), *bad, A, need, None) == 1
    assert f(ctypes.byref(_shape(T=0)), *([None] * 10), None, 0, None) == 0
    assert _lib.w4a16_workspace(4, 200, 128, 8, 2) == 0              # invalid shape -> 0
    if _no_gpu():
        assert f(ctypes.byref(s), *ok, A, need, None) == 6


@needs_lib
def test_w4a8_validation():
    f = LIB.moe_grouped_w4a8_ffn
    s = _shape()
    need = _lib.w4a8_workspace(4, 256, 128, 8, 2)
    # xq, xs; h float32; hq, hs (each 256-byte aligned)
    assert need == 1024 + 256 + 4096 + 1024 + 256
    ok = [A] * 10
    assert f(ctypes.byref(_shape(H=192)), *ok, None, A, need, None) == 2     # H % 128
    assert f(ctypes.byref(_shape(I=64)), *ok, None, A, need, None) == 2      # I % 128
    assert f(ctypes.byref(_shape(k=9)), *ok, None, A, need, None) == 2
    assert f(ctypes.byref(_shape(H=16512)), *ok, None, A, need, None) == 2   # H > MOE_MAX_DIM
    assert f(None, *ok, None, A, need, None) == 1
    assert f(ctypes.byref(s), *ok, None, A, need - 1, None) == 4
    bad = list(ok)
    bad[9] = None                                                        # y
    assert f(ctypes.byref(s), *bad, None, A, need, None) == 1
    dbg = _lib.MoeW4A8Debug(A, A, MIS, None)
    assert f(ctypes.byref(s), *ok, ctypes.byref(dbg), A, need, None) == 3
    assert f(ctypes.byref(_shape(T=0)), *([None] * 10), None, None, 0, None) == 0
    assert _lib.w4a8_workspace(4, 192, 128, 8, 2) == 0
    if _no_gpu():
        assert f(ctypes.byref(s), *ok, None, A, need, None) == 6


def test_w8a8_validation():
    f = LIB.moe_grouped_w8a8_ffn
    s = _shape(H=208, I=48)          # W8A8 needs multiples of 16 only
    need = _lib.w8a8_workspace(4, 208, 48, 8, 2)
    assert need > 0
    ok = [A] * 10
    assert f(ctypes.byref(_shape(H=100)), *ok, None, A, need, None) == 2
    assert f(ctypes.byref(_shape(H=208, I=40)), *ok, None, A, need, None) == 2
    assert _lib.w8a8_workspace(4, 200, 48, 8, 2) == 0      # H % 16 != 0: no workspace size
    assert f(ctypes.byref(s), *ok, None, A, need - 1, None) == 4
    dbg = _lib.MoeW8A8Debug(A, MIS, None, None, None, None)
    assert f(ctypes.byref(s), *ok, ctypes.byref(dbg), A, need, None) == 3
    if _no_gpu():
        assert f(ctypes.byref(s), *ok, None, A, need, None) == 6


@needs_lib
def test_combine_validation():
    f = LIB.moe_combine
    assert f(A, A, A, 4, 100, 2, A, None) == 2      # H % 8
    assert f(A, A, A, 4, 256, 0, A, None) == 2
    assert f(A, A, A, -1, 256, 2, A, None) == 1
    assert f(A, None, A, 4, 256, 2, A, None) == 1
    assert f(A, A, A, 4, 256, 2, MIS, None) == 3
    assert f(None, None, None, 0, 256, 2, None, None) == 0
    if _no_gpu():
        assert f(A, A, A, 4, 256, 2, A, None) == 6


@needs_lib
def test_binding_raises_moe_error():
    import torch
    t = torch.empty((4, 8))
    out = torch.empty((4, 9))
    with pytest.raises(_lib.MoeError) as ei:
        _lib.route_topk(t, 9, out, out, stream=0)
    assert ei.value.status == 2
    with pytest.raises(ValueError):          # buffer smaller than the call needs
        _lib.route_topk(t, 2, torch.empty(7), out, stream=0)


@needs_lib
def test_layer_w4a16_validation():
    f = LIB.moe_layer_w4a16
    s = _shape()
    need = _lib.layer_w4a16_workspace(4, 256, 128, 8, 2)
    assert need > 0
    ok = [A] * 15       # logits, x, w13, s13, w2, s2, ids, w, offsets, sorted, pos, active, n_active, y, out
    assert f(ctypes.byref(_shape(H=200)), *ok, A, need, None) == 2
    assert f(ctypes.byref(s), *ok, A, need - 1, None) == 4
    bad = list(ok)
    bad[0] = MIS
    assert f(ctypes.byref(s), *bad, A, need, None) == 3
    bad[0] = None
    assert f(ctypes.byref(s), *bad, A, need, None) == 1
    if _no_gpu():
        assert f(ctypes.byref(s), *ok, A, need, None) == 6
    # the Python wrapper marshals the same 20 arguments
    import torch
    dummy = torch.empty(64, dtype=torch.uint8)
    with pytest.raises(_lib.MoeError):
        _lib.layer_w4a16((4, 200, 128, 8, 2), *([dummy] * 15), dummy, stream=0)


@needs_lib
@pytest.mark.parametrize("args,status", [
    ((A, B, -1, 256, 8, A), 1),          # T < 0
    ((A, B, 2, 96, 8, A), 2),            # H not a multiple of 64
    ((A, B, 2, 0, 8, A), 2),             # H = 0
    ((A, B, 2, 256, 0, A), 2),           # E = 0
    ((A, B, 2, 256, 1025, A), 2),        # E > MOE_MAX_EXPERTS
    ((None, B, 2, 256, 8, A), 1),        # null x
    ((A, None, 2, 256, 8, A), 1),        # null router rows
    ((A, B, 2, 256, 8, None), 1),        # null logits
    ((MIS, B, 2, 256, 8, A), 3),         # misaligned x
    ((A, B, 0, 256, 8, None), 0),        # empty batch: nothing to check or launch
])
def test_router_logits_validation(args, status):
    assert LIB.moe_router_logits(*args, None) == status
    if status:
        assert LIB.moe_last_error()


@needs_lib
def test_expert_telemetry_validation():
    f = LIB.moe_expert_counts_accumulate
    assert f(A, 9, -1, 8, A, None) == 1                  # L < 0
    assert f(A, 9, 2, 0, A, None) == 2                   # E < 1
    assert f(A, 9, 2, 1025, A, None) == 2                # E > MOE_MAX_EXPERTS
    assert f(A, 8, 2, 8, A, None) == 2                   # stride < E + 1
    assert f(None, 9, 0, 8, None, None) == 0             # nothing to do
    assert f(None, 9, 2, 8, A, None) == 1
    assert f(A, 9, 2, 8, MIS, None) == 3
    h = LIB.moe_expert_hot_rank
    assert h(A, 1, 8, 9, A, None) == 2                   # n > E
    assert h(A, 1, 8, -1, A, None) == 2
    assert h(A, -1, 8, 2, A, None) == 1
    assert h(None, 3, 8, 0, None, None) == 0             # n = 0: nothing to do
    assert h(A, 3, 8, 2, None, None) == 1
    if _no_gpu():
        assert f(A, 9, 2, 8, A, None) == 6
        assert h(A, 3, 8, 2, A, None) == 6


@needs_lib
def test_layer_w4a16_noalloc_validation():
    """The no-allocation layer entry: shapes whose workspace exceeds the static
    scratch are refused before anything else; then the usual checks."""
    f = LIB.moe_layer_w4a16_noalloc
    ok = [A] * 15
    big = _shape(T=4096, H=2048, I=768, E=128, k=8)
    assert _lib.layer_w4a16_workspace(4096, 2048, 768, 128, 8) > 8 << 20
    assert f(ctypes.byref(big), *ok, None) == 4
    assert b"static scratch" in LIB.moe_last_error()
    s = _shape()
    assert f(ctypes.byref(_shape(H=200)), *ok, None) == 2
    bad = list(ok)
    bad[1] = MIS
    assert f(ctypes.byref(s), *bad, None) == 3
    bad[1] = None
    assert f(ctypes.byref(s), *bad, None) == 1
    if _no_gpu():
        assert f(ctypes.byref(s), *ok, None) == 6


@needs_lib
def test_library_leaves_no_kernel_symbol_undefined():
    """Every launch stub the host code references is defined in libmoe.so (a
    kernel whose host stub the compiler drops still links into a shared
    library, and fails only when the library is loaded)."""
    import shutil
    import subprocess
    if shutil.which("nm") is None:
        pytest.skip("nm not available")
    out = subprocess.run(["nm", "-C", "-u", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    missing = [ln for ln in out.splitlines() if "moe::" in ln]
    assert not missing, "\n".join(missing)
