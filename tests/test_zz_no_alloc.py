"""The no-allocation layer entry point (moe_layer_w4a16_noalloc, workspace in
the library's static device scratch) against the workspace entry point
(moe_layer_w4a16) through the C ABI: every output bit for bit, on two calls in
a row whose second is smaller (a prefill-sized batch, then a decode batch that
takes the fused kernels), and the refusal of a shape whose workspace exceeds
the scratch."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth  # noqa: E402
from gpu_util import stage_weights, to_dev, to_np  # noqa: E402

pytestmark = pytest.mark.gpu

KEYS = ("ids", "w", "offsets", "sorted_slot", "slot_pos", "active", "n_active", "y", "out")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_expert_top_amd as moe
    moe.load()


def _outputs(b):
    torch.cuda.synchronize()
    R = b.T * b.k
    n = int(to_np(b.n_active)[0])
    return {"ids": to_np(b.ids), "w": to_np(b.w).view(np.uint32),
            "offsets": to_np(b.offsets)[:b.E + 1], "sorted_slot": to_np(b.sorted_slot)[:R],
            "slot_pos": to_np(b.slot_pos)[:R], "active": to_np(b.active)[:n], "n_active": n,
            "y": to_np(b.y)[:R].view(np.uint32), "out": to_np(b.out).view(np.uint32)}


def _both(wl, unit):
    import quantized_moe_expert_top_amd as moe
    x, L = to_dev(synth.x_bf16(wl, unit)), to_dev(synth.router_logits(wl, unit))
    wts = stage_weights(wl, unit)
    ref = moe.LayerBuffers.alloc(wl.T, wl.H, wl.I, wl.E, wl.k, "w4a16")
    moe.moe_layer(ref, x, L, wts)
    want = _outputs(ref)
    got = moe.LayerBuffers.alloc(wl.T, wl.H, wl.I, wl.E, wl.k, "w4a16")
    for t in (got.y, got.out):
        t.fill_(float("nan"))
    moe.layer_w4a16_noalloc((wl.T, wl.H, wl.I, wl.E, wl.k), L, x, *wts, got.ids, got.w,
                            got.offsets, got.sorted_slot, got.slot_pos, got.active, got.n_active,
                            got.y, got.out)
    return want, _outputs(got)


def test_noalloc_matches_workspace_entry_on_two_calls():
    first = synth.Workload("noalloc_t64", 601, 64, 2048, 768, 128, 8, "w4a16", "normal", 1)
    second = first.with_(name="noalloc_t2", T=2)      # smaller: the fused decode kernels
    for wl in (first, second):
        print("[case] noalloc", wl.name, (wl.T, wl.H, wl.I, wl.E, wl.k), flush=True)
        want, got = _both(wl, 0)
        for key in KEYS:
            np.testing.assert_array_equal(got[key], want[key], err_msg=f"{wl.name}: {key}")


def test_noalloc_refuses_a_shape_beyond_the_scratch():
    """Through the C ABI: MOE_EWORKSPACE and its message, nothing launched."""
    import ctypes

    import quantized_moe_expert_top_amd as moe
    from quantized_moe_expert_top_amd import _lib
    T, H, I, E, k = 4096, 2048, 768, 128, 8         # h alone is 50 MB
    assert moe.layer_w4a16_workspace(T, H, I, E, k) > 8 << 20
    d = torch.empty(16, dtype=torch.uint8, device="cuda")
    lib = _lib.load()
    shape = _lib.MoeShape(T, H, I, E, k)
    status = lib.moe_layer_w4a16_noalloc(ctypes.byref(shape), *([d.data_ptr()] * 15), None)
    assert status == 4
    assert b"static scratch" in lib.moe_last_error()
