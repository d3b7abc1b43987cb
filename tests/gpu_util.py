"""Helpers shared by the GPU parity tests: staging numpy inputs on the device,
running the layer through the C ABI, and the float tolerance check."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth
import quantized_moe_expert_top_amd as moe

# Float tolerance for layer outputs: relative L2 over the whole output and a
# per-element bound relative to the oracle row's rms (a zero row must be 0).
REL_L2 = 5e-3
ELEM_RMS = 2e-2


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint8:
        return torch.from_numpy(a).cuda()
    return torch.from_numpy(a).cuda()


def to_np(t: torch.Tensor, dtype=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    return a.view(dtype) if dtype is not None else a


def bf16_np_to_f64(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_to_f64(to_np(t).view(np.uint16))


def assert_close(got: np.ndarray, ref: np.ndarray, what: str,
                 rel_l2: float = REL_L2, elem: float = ELEM_RMS) -> dict:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = got - ref
    nref = np.linalg.norm(ref)
    rl2 = np.linalg.norm(err) / nref if nref > 0 else np.linalg.norm(err)
    rms = np.sqrt(np.mean(ref ** 2, axis=-1, keepdims=True))
    zero_rows = rms[..., 0] == 0
    assert np.all(got[zero_rows] == 0), f"{what}: a zero oracle row is not exactly zero"
    lim = elem * np.where(rms > 0, rms, 1.0)
    worst = float(np.max(np.abs(err) / lim)) if err.size else 0.0
    assert rl2 <= rel_l2, f"{what}: relative L2 {rl2:.3e} > {rel_l2}"
    assert worst <= 1.0, f"{what}: element error {worst * elem:.3e} x rms(row) > {elem}"
    return {"rel_l2": rl2, "worst_elem_over_rms": worst * elem}


def expert_getter_w4(wl, unit):
    return lambda e: synth.expert_w4(wl, unit, e, "w13") + synth.expert_w4(wl, unit, e, "w2")


def expert_getter_w8(wl, unit):
    return lambda e: synth.expert_w8(wl, unit, e, "w13") + synth.expert_w8(wl, unit, e, "w2")


def stage_weights(wl, unit, experts=None):
    if wl.fmt in ("w4a16", "w4a8"):
        arrs = synth.layer_w4(wl, unit, experts)
    else:
        arrs = synth.layer_w8(wl, unit)
    return tuple(to_dev(a) for a in arrs)


def run_layer(wl, x_bits, logits, weights, debug=False):
    """Whole layer through the five entry points; returns numpy results."""
    b = moe.LayerBuffers.alloc(wl.T, wl.H, wl.I, wl.E, wl.k, wl.fmt)
    dbg = None
    if debug and wl.fmt == "w8a8":
        R = wl.T * wl.k
        dbg = {
            "xq": torch.empty((wl.T, wl.H), dtype=torch.int8, device="cuda"),
            "xs": torch.empty(wl.T, dtype=torch.float32, device="cuda"),
            "acc13": torch.empty((R, 2 * wl.I), dtype=torch.int32, device="cuda"),
            "hq": torch.empty((R, wl.I), dtype=torch.int8, device="cuda"),
            "hs": torch.empty(R, dtype=torch.float32, device="cuda"),
            "acc2": torch.empty((R, wl.H), dtype=torch.int32, device="cuda"),
        }
    if debug and wl.fmt == "w4a8":
        R = wl.T * wl.k
        dbg = {
            "xq": torch.empty((wl.T, wl.H), dtype=torch.int8, device="cuda"),
            "xs": torch.empty(wl.T, dtype=torch.float32, device="cuda"),
            "hq": torch.empty((R, wl.I), dtype=torch.int8, device="cuda"),
            "hs": torch.empty(R, dtype=torch.float32, device="cuda"),
        }
    moe.moe_forward(b, to_dev(x_bits), to_dev(logits), weights, debug=dbg)
    torch.cuda.synchronize()
    R = wl.T * wl.k
    n_act = int(to_np(b.n_active)[0])
    res = {
        "ids": to_np(b.ids),
        "w": to_np(b.w),
        "expert_offsets": to_np(b.offsets),
        "sorted_slot": to_np(b.sorted_slot)[:R],
        "slot_pos": to_np(b.slot_pos)[:R],
        "n_active": n_act,
        "active": to_np(b.active)[:n_act],
        "y": to_np(b.y)[:R].astype(np.float64) if R else np.zeros((0, wl.H)),
        "out": to_np(b.out).astype(np.float64),
        "y_bits": to_np(b.y)[:R].copy(),
        "out_bits": to_np(b.out).view(np.uint32).copy(),
    }
    if dbg:
        for kk, v in dbg.items():
            res[kk] = to_np(v)
    return res


def check_routing_and_perm(res, ref):
    np.testing.assert_array_equal(res["ids"], ref["ids"])
    np.testing.assert_allclose(res["w"], ref["w"], rtol=0, atol=1e-6)
    p = ref["perm"]
    np.testing.assert_array_equal(res["expert_offsets"], p["expert_offsets"])
    np.testing.assert_array_equal(res["sorted_slot"], p["sorted_slot"])
    np.testing.assert_array_equal(res["slot_pos"], p["slot_pos"])
    assert res["n_active"] == p["n_active"]
    np.testing.assert_array_equal(res["active"], p["active"])
