"""GPU parity: every step of the layer through the C ABI against the CPU oracle
on the same seeded inputs. Integers (ids, permutation, W8A8 codes and int32
accumulators) bit-exact; floats within the layer tolerance."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import synth  # noqa: E402
from gpu_util import (assert_close, check_routing_and_perm, expert_getter_w4,  # noqa: E402
                      expert_getter_w8, run_layer, stage_weights, to_dev, to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_expert_top_amd as moe
    moe.load()


def _say(*a):
    print("[case]", *a, flush=True)


# ----------------------------------------------------------------- routing --
def _route_gpu(L, k):
    import quantized_moe_expert_top_amd as moe
    T, E = L.shape
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.route_topk(to_dev(np.ascontiguousarray(L, np.float32)), k, ids, w)
    torch.cuda.synchronize()
    return to_np(ids), to_np(w)


@pytest.mark.parametrize("name,unit", [("tiny", 0), ("decode_t2", 0), ("decode_t2", 7),
                                       ("prefill_t512", 0), ("w8a8_t4096", 0),
                                       ("decode_large", 3)])
def test_route_workloads(name, unit):
    wl = synth.workload(name)
    _say("route", name, unit, wl.T, wl.E, wl.k)
    L = synth.router_logits(wl, unit)
    ids, w = _route_gpu(L, wl.k)
    rids, rw = oracle.route_topk(L, wl.k)
    np.testing.assert_array_equal(ids, rids)
    np.testing.assert_allclose(w, rw, rtol=0, atol=1e-6)


def test_route_hand_cases_and_ties():
    import json
    import os
    cases = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "route_hand.json")))
    for c in cases["cases"]:
        L = np.array(c["logits"], np.float32)
        ids, w = _route_gpu(L, c["k"])
        np.testing.assert_array_equal(ids, c["ids"])
        np.testing.assert_allclose(w, c["w"], rtol=0, atol=1e-6)


@pytest.mark.parametrize("T,E,k", [(33, 1024, 32), (64, 1, 1), (17, 256, 8), (5, 64, 64 // 2),
                                   (9, 300, 7)])
def test_route_forced_ties_and_extremes(T, E, k):
    rng = np.random.default_rng(T * 7 + E)
    L = rng.integers(-2, 3, size=(T, E)).astype(np.float32)
    L[L == 0] = np.where(rng.random(np.count_nonzero(L == 0)) < 0.5, 0.0, -0.0)
    _say("route ties", T, E, k)
    ids, w = _route_gpu(L, k)
    rids, rw = oracle.route_topk(L, k)
    np.testing.assert_array_equal(ids, rids)
    np.testing.assert_allclose(w, rw, rtol=0, atol=1e-6)


# ------------------------------------------------------------- permutation --
def _permute_gpu(ids, E):
    import quantized_moe_expert_top_amd as moe
    T, k = ids.shape
    R = T * k
    d = lambda n: torch.full((max(n, 1),), -7, dtype=torch.int32, device="cuda")  # noqa: E731
    off, ss, sp, act, na = d(E + 1), d(R), d(R), d(min(E, R)), d(1)
    ws = torch.empty(max(moe.permute_workspace(T, E, k), 16), dtype=torch.uint8, device="cuda")
    moe.permute(to_dev(np.ascontiguousarray(ids, np.int32)), E, off, ss, sp, act, na, ws)
    torch.cuda.synchronize()
    n = int(to_np(na)[0])
    return {"expert_offsets": to_np(off)[:E + 1], "sorted_slot": to_np(ss)[:R],
            "slot_pos": to_np(sp)[:R], "active": to_np(act)[:n], "n_active": n}


def _random_ids(T, E, k, seed, skew=0.0):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)) - skew * np.log(np.arange(1, E + 1))
    return oracle.route_topk(logits.astype(np.float32), k)[0]


@pytest.mark.parametrize("T,E,k,skew", [(16, 8, 2, 0), (2, 128, 8, 0), (129, 128, 8, 0),
                                        (4096, 128, 8, 0), (4096, 128, 8, 2.0), (64, 1024, 32, 0),
                                        (1, 1, 1, 0), (1000, 3, 3, 0), (300, 256, 8, 1.1),
                                        (1024, 128, 8, 0.5), (2731, 64, 3, 0), (20, 512, 32, 0),
                                        # the one-wave offsets scan up to E 256 and R < 65536,
                                        # the block scan past either bound
                                        (8191, 128, 8, 0), (8192, 128, 8, 0), (100, 257, 4, 0)])
def test_permute_matches_oracle(T, E, k, skew):
    ids = _random_ids(T, E, k, T + E, skew)
    _say("permute", T, E, k, skew)
    got = _permute_gpu(ids, E)
    ref = oracle.permute(ids, E)
    for key in ("expert_offsets", "sorted_slot", "slot_pos", "active"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    assert got["n_active"] == ref["n_active"]


def test_permute_empty_batch():
    got = _permute_gpu(np.zeros((0, 4), np.int32), 16)
    assert np.all(got["expert_offsets"] == 0) and got["n_active"] == 0


# ----------------------------------------------------------------- combine --
@pytest.mark.parametrize("k", [1, 5, 8, 13, 16, 32])
def test_combine_matches_oracle(k):
    # k below, at and past the kernel's batch of eight picks, with a partial
    # batch after full ones (13) and several full batches (16, 32)
    import quantized_moe_expert_top_amd as moe
    rng = np.random.default_rng(1 + k)
    T, H = 77, 520
    y = rng.standard_normal((T * k, H)).astype(np.float32)
    slot_pos = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    moe.combine(to_dev(y), to_dev(slot_pos), to_dev(w), out)
    torch.cuda.synchronize()
    ref = oracle.combine(y.astype(np.float64), slot_pos, w.astype(np.float64))
    np.testing.assert_allclose(to_np(out), ref, rtol=1e-5, atol=1e-5)


# ------------------------------------------------------------ W4A16 layer --
def _w4_layer_case(wl, unit=0, logits=None, only_routed=True):
    x = synth.x_bf16(wl, unit)
    L = synth.router_logits(wl, unit) if logits is None else logits
    ref = oracle.moe_layer_w4a16(x, L, wl.k, expert_getter_w4(wl, unit))
    experts = ref["perm"]["active"] if only_routed else None
    _say("w4a16 layer", wl.name, unit, (wl.T, wl.H, wl.I, wl.E, wl.k))
    res = run_layer(wl, x, L, stage_weights(wl, unit, experts))
    check_routing_and_perm(res, ref)
    s1 = assert_close(res["y"], ref["y"], "y")
    s2 = assert_close(res["out"], ref["out"], "out")
    return res, ref, s1, s2


CUSTOM_W4 = [
    # name, wid, T, H, I, E, k : ragged and edge shapes on both kernels
    ("gemv_t1", 101, 1, 256, 128, 8, 2),
    ("gemv_t3_ragged", 102, 3, 384, 384, 16, 4),       # K=384: 12 chunks -> 4 lanes per row
    ("gemv_t4", 103, 4, 1280, 640, 32, 6),
    ("mfma_t5", 104, 5, 256, 128, 8, 2),
    ("mfma_t37_ragged", 105, 37, 640, 384, 12, 3),     # 5 groups, I not a multiple of 256
    ("mfma_t300_dense", 106, 300, 256, 256, 4, 2),     # >64 rows per expert: m-tile loop
    ("e1_k1", 107, 9, 256, 128, 1, 1),
    ("k_equals_e", 108, 6, 256, 128, 4, 4),
]


@pytest.mark.parametrize("case", CUSTOM_W4, ids=[c[0] for c in CUSTOM_W4])
def test_w4a16_custom_shapes(case):
    name, wid, T, H, I, E, k = case
    wl = synth.Workload(name, wid, T, H, I, E, k, "w4a16", "normal", 1)
    _w4_layer_case(wl, only_routed=False)


@pytest.mark.parametrize("name,unit", [("tiny", 0), ("decode_t2", 0), ("decode_t2", 31),
                                       ("prefill_t512", 0), ("prefill_t512", 5)])
def test_w4a16_workload_layers(name, unit):
    wl = synth.workload(name)
    _w4_layer_case(wl, unit)


def test_w4a16_decode_large_steps():
    wl = synth.workload("decode_large")
    for step in (0, 9):
        _w4_layer_case(wl, step)


@pytest.mark.parametrize("T", [4, 300])
def test_w4a16_all_tokens_one_expert(T):
    """Degenerate routing: every token's top pick is expert 3 (one expert holds T rows)."""
    wl = synth.Workload(f"skew_t{T}", 120 + T, T, 512, 256, 16, 2, "w4a16", "none", 1)
    L = synth.router_logits(wl, 0).astype(np.float64)
    L[:, 3] += 50.0
    _w4_layer_case(wl, logits=L.astype(np.float32), only_routed=False)


def test_w4a16_zero_inputs_give_zero():
    wl = synth.Workload("zeros", 130, 8, 256, 128, 8, 2, "w4a16", "none", 1)
    x = np.zeros((wl.T, wl.H), np.uint16)
    L = synth.router_logits(wl, 0)
    res = run_layer(wl, x, L, stage_weights(wl, 0))
    assert np.all(res["out"] == 0.0)
    for T in (2, 8):   # down codes all 8 -> exact zeros, on both kernels
        wl2 = wl.with_(T=T)
        w13, s13, w2, s2 = synth.layer_w4(wl2, 0)
        w2[:] = 0x88
        res = run_layer(wl2, synth.x_bf16(wl2, 0), synth.router_logits(wl2, 0),
                        tuple(to_dev(a) for a in (w13, s13, w2, s2)))
        assert np.all(res["out"] == 0.0)


def test_w4a16_deterministic():
    for name in ("tiny", "prefill_t512", "decode_t2"):
        wl = synth.workload(name)
        x, L = synth.x_bf16(wl, 0), synth.router_logits(wl, 0)
        wts = stage_weights(wl, 0)
        a = run_layer(wl, x, L, wts)
        b = run_layer(wl, x, L, wts)
        np.testing.assert_array_equal(a["y_bits"], b["y_bits"])
        np.testing.assert_array_equal(a["out_bits"], b["out_bits"])


# ------------------------------------------------------------- W8A8 layer --
def _check_w8a8(res, ref, w2_getter):
    np.testing.assert_array_equal(res["xq"], ref["xq"])
    np.testing.assert_array_equal(res["xs"].view(np.uint32), ref["xs"].view(np.uint32))
    np.testing.assert_array_equal(res["acc13"], ref["acc13"])
    # h codes: decided in float32 on both sides from float32 h that differ by
    # rounding only; a code may differ by one step, and only at a .5 boundary
    dq = res["hq"].astype(np.int32) - ref["hq"].astype(np.int32)
    assert np.all(np.abs(dq) <= 1)
    assert np.count_nonzero(dq) <= 1e-3 * dq.size + 1
    np.testing.assert_allclose(res["hs"], ref["hs"], rtol=1e-5, atol=0)
    if np.count_nonzero(dq):
        v = np.abs(ref["h"] / np.where(ref["hs"] > 0, ref["hs"], 1)[:, None])
        near = np.abs(v - np.floor(v) - 0.5) < 1e-3
        assert np.all(near[dq != 0])
    # down accumulators: exact where the codes agree; elsewhere the difference
    # is exactly the integer product of the code difference
    same = ~np.any(dq != 0, axis=1)
    np.testing.assert_array_equal(res["acc2"][same], ref["acc2"][same])
    off = ref["perm"]["expert_offsets"]
    for p in np.nonzero(~same)[0]:
        e = int(np.searchsorted(off, p, side="right") - 1)
        w2 = w2_getter(e)
        want = ref["acc2"][p] + w2.astype(np.int64) @ dq[p].astype(np.int64)
        np.testing.assert_array_equal(res["acc2"][p], want)
    s1 = assert_close(res["y"], ref["y"], "y")
    s2 = assert_close(res["out"], ref["out"], "out")
    return s1, s2


def _w8_case(wl, unit=0):
    x = synth.x_bf16(wl, unit)
    L = synth.router_logits(wl, unit)
    get = expert_getter_w8(wl, unit)
    ref = oracle.moe_layer_w8a8(x, L, wl.k, get)
    _say("w8a8 layer", wl.name, unit, (wl.T, wl.H, wl.I, wl.E, wl.k))
    res = run_layer(wl, x, L, stage_weights(wl, unit), debug=True)
    check_routing_and_perm(res, ref)
    return _check_w8a8(res, ref, lambda e: get(e)[2])


CUSTOM_W8 = [
    ("w8_small", 201, 64, 256, 128, 8, 2),
    ("w8_ragged", 202, 45, 192, 320, 6, 3),   # K=192/320: not multiples of 128
    ("w8_t1", 203, 1, 128, 64, 4, 1),
    ("w8_many_rows", 204, 700, 256, 128, 4, 2),   # >128 rows per expert
    ("w8_e1024", 206, 40, 256, 128, 1024, 32),    # most experts hold one row
    ("w8_k_tail_16_48", 207, 37, 208, 176, 8, 2),  # H % 64 = 16, I % 64 = 48: zero-filled tails
    ("w8_k_tail_32", 208, 20, 160, 96, 8, 3),       # H % 64 = I % 64 = 32
]


@pytest.mark.parametrize("case", CUSTOM_W8, ids=[c[0] for c in CUSTOM_W8])
def test_w8a8_custom_shapes(case):
    name, wid, T, H, I, E, k = case
    _w8_case(synth.Workload(name, wid, T, H, I, E, k, "w8a8", "none", 1))


def test_w8a8_full_layer_t4096():
    _w8_case(synth.workload("w8a8_t4096"), 1)


def test_w8a8_zero_token_row():
    wl = synth.Workload("w8_zero_row", 205, 12, 256, 128, 8, 2, "w8a8", "none", 1)
    x = synth.x_bf16(wl, 0)
    x[5] = 0
    L = synth.router_logits(wl, 0)
    get = expert_getter_w8(wl, 0)
    ref = oracle.moe_layer_w8a8(x, L, wl.k, get)
    res = run_layer(wl, x, L, stage_weights(wl, 0), debug=True)
    assert res["xs"][5] == 0 and np.all(res["xq"][5] == 0)
    assert np.all(res["out"][5] == 0)
    _check_w8a8(res, ref, lambda e: get(e)[2])


# ------------------------------------------------------------- W4A8 layer --
def _w4a8_down_from(hq, hs, perm, get):
    """The down projection of the oracle applied to the kernel's own h codes
    and scales, with a per-element bound on float32 rounding: the G group
    terms are summed in float32 (each term rounded once, every partial sum
    once), then scaled by the row scale."""
    off = perm["expert_offsets"]
    R = hq.shape[0]
    H = None
    y = bound = None
    for e in perm["active"]:
        a, b = int(off[e]), int(off[e + 1])
        _, _, w2, s2 = get(int(e))
        Q2 = oracle.unpack_int4(w2).astype(np.int64) - oracle.ZERO_POINT
        if y is None:
            H = Q2.shape[0]
            y = np.zeros((R, H))
            bound = np.zeros((R, H))
        terms = oracle.group_int_dots(hq[a:b], Q2) * oracle.fp16_to_f64(s2)[None, :, :]
        G = terms.shape[2]
        hs_e = hs[a:b].astype(np.float64)[:, None]
        y[a:b] = terms.sum(axis=2) * hs_e
        bound[a:b] = (G + 2) * 2.0 ** -24 * np.abs(terms).sum(axis=2) * hs_e
    return y, bound


def _check_w4a8(res, ref, get):
    np.testing.assert_array_equal(res["xq"], ref["xq"])
    np.testing.assert_array_equal(res["xs"].view(np.uint32), ref["xs"].view(np.uint32))
    # h: float32 sums of group terms against the float64 of the oracle; a code
    # may differ by one step, only where h / hs lies at a .5 boundary
    dq = res["hq"].astype(np.int32) - ref["hq"].astype(np.int32)
    assert np.all(np.abs(dq) <= 1)
    assert np.count_nonzero(dq) <= 1e-3 * dq.size + 1
    np.testing.assert_allclose(res["hs"], ref["hs"], rtol=1e-5, atol=0)
    if np.count_nonzero(dq):
        v = np.abs(ref["h"] / np.where(ref["hs"] > 0, ref["hs"], 1)[:, None])
        near = np.abs(v - np.floor(v) - 0.5) < 2e-3
        assert np.all(near[dq != 0])
    # down: exact integer group dots of the kernel's own codes, so y may differ
    # from that float64 value by float32 rounding only
    R = res["hq"].shape[0]
    if R == 0:
        return None
    want, bound = _w4a8_down_from(res["hq"], res["hs"], ref["perm"], get)
    err = np.abs(res["y"] - want)
    assert np.all(err <= bound + 1e-30), float(np.max(err - bound))
    # against the oracle end to end: rows whose h codes all agree element by
    # element; a row with a boundary flip moves by that one code step times a
    # weight column, which the check above already holds exactly, so there
    # the layer is compared as a whole (relative L2)
    same = ~np.any(dq != 0, axis=1)
    s1 = assert_close(res["y"][same], ref["y"][same], "y")
    assert_close(res["y"], ref["y"], "y", elem=np.inf)
    tok_same = np.ones(res["out"].shape[0], bool)
    tok_same[ref["perm"]["sorted_slot"][~same] // ref["ids"].shape[1]] = False
    s2 = assert_close(res["out"][tok_same], ref["out"][tok_same], "out")
    assert_close(res["out"], ref["out"], "out", elem=np.inf)
    out_own = oracle.combine(want, ref["perm"]["slot_pos"], ref["w"])
    assert_close(res["out"], out_own, "out (own codes)")
    return s1, s2


def _w4a8_case(wl, unit=0, x=None, weights=None):
    x = synth.x_bf16(wl, unit) if x is None else x
    L = synth.router_logits(wl, unit)
    get = expert_getter_w4(wl, unit)
    ref = oracle.moe_layer_w4a8(x, L, wl.k, get)
    _say("w4a8 layer", wl.name, unit, (wl.T, wl.H, wl.I, wl.E, wl.k))
    wts = stage_weights(wl, unit, np.unique(ref["ids"])) if weights is None else weights
    res = run_layer(wl, x, L, wts, debug=True)
    check_routing_and_perm(res, ref)
    _check_w4a8(res, ref, get)
    return res, ref


CUSTOM_W4A8 = [
    ("w4a8_small", 301, 64, 256, 128, 8, 2),
    ("w4a8_ragged", 302, 45, 384, 256, 6, 3),      # 3 groups of x: the ring wraps mid-row
    ("w4a8_t1", 303, 1, 128, 128, 4, 1),           # one group per row
    ("w4a8_many_rows", 304, 700, 256, 128, 4, 2),  # many 32-row tiles per expert
    ("w4a8_wide", 305, 33, 640, 384, 16, 4),       # partial 256-column down tile
    ("w4a8_tall", 308, 301, 384, 384, 4, 3),       # 64-row tiles, ragged last tile, 3 groups
    ("w4a8_k3072", 310, 24, 3072, 256, 8, 2),      # 96 KiB resident tile: one block per CU
    ("w4a8_deep", 309, 16, 4864, 128, 8, 2),       # long K: many groups per tile
    ("w4a8_e1024", 311, 40, 256, 128, 1024, 32),   # most experts hold one row
]


def test_int4_gemms_at_the_largest_dim():
    """H = MOE_MAX_DIM on the MFMA paths with 64-row tiles (the scale strips
    take the most LDS there): W4A16 and W4A8 against the oracle. I = 512: at
    this H the bf16 rounding of h alone (W4A16) puts single y elements at
    1.5% of the row rms (2.1% with I = 128, where y sums only 128 terms)."""
    wl16 = synth.Workload("w4_maxdim", 312, 64, 16384, 512, 1, 1, "w4a16", "none", 1)
    x, L = synth.x_bf16(wl16, 0), synth.router_logits(wl16, 0)
    ref = oracle.moe_layer_w4a16(x, L, 1, expert_getter_w4(wl16, 0))
    _say("w4a16 max dim")
    res = run_layer(wl16, x, L, stage_weights(wl16, 0))
    check_routing_and_perm(res, ref)
    assert_close(res["y"], ref["y"], "y")
    assert_close(res["out"], ref["out"], "out")
    _say("w4a8 max dim")
    _w4a8_case(wl16.with_(name="w4a8_maxdim", fmt="w4a8"))


@pytest.mark.parametrize("case", CUSTOM_W4A8, ids=[c[0] for c in CUSTOM_W4A8])
def test_w4a8_custom_shapes(case):
    name, wid, T, H, I, E, k = case
    _w4a8_case(synth.Workload(name, wid, T, H, I, E, k, "w4a8", "none", 1))


def test_w4a8_prefill_layer_t512():
    _w4a8_case(synth.workload("w4a8_t512"), 5)


def test_w4a8_zero_row_and_zero_weights():
    wl = synth.Workload("w4a8_zero", 306, 20, 256, 256, 8, 2, "w4a8", "none", 1)
    x = synth.x_bf16(wl, 0)
    x[7] = 0
    res, _ = _w4a8_case(wl, 0, x=x)
    assert res["xs"][7] == 0 and np.all(res["xq"][7] == 0)
    assert np.all(res["out"][7] == 0)
    # every down code at the zero point (byte 0x88): y and out exactly zero
    L = synth.router_logits(wl, 0)
    w13, s13, w2, s2 = stage_weights(wl, 0)
    w2.fill_(0x88)
    r = run_layer(wl, x, L, (w13, s13, w2, s2), debug=True)
    assert np.all(r["y_bits"] == 0) and np.all(r["out_bits"] == 0)


def test_w4a8_deterministic():
    wl = synth.Workload("w4a8_det", 307, 96, 512, 256, 16, 4, "w4a8", "none", 1)
    x, L = synth.x_bf16(wl, 0), synth.router_logits(wl, 0)
    wts = stage_weights(wl, 0)
    a = run_layer(wl, x, L, wts)
    b = run_layer(wl, x, L, wts)
    np.testing.assert_array_equal(a["y_bits"], b["y_bits"])
    np.testing.assert_array_equal(a["out_bits"], b["out_bits"])


def _sweep_cases(n=12, seed=2026, tag="sweep", wid0=400):
    """Seeded random layer shapes over the three formats, small enough for the
    float64 oracle: T past the decode GEMV (MFMA paths), W4 dims multiples of
    128, W8A8 dims multiples of 16, E from 1 to 64, k up to min(E, 8), skewed
    router logits for the W4 formats. W4A16 takes I >= 256: its h is bf16 (the
    MFMA operand), and with I = 128 the rounding of h alone moves single y
    elements past 2% of the row rms (2.14% at H 1280, computed on the CPU
    from the float64 h), whatever the kernel does."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fmt = ("w4a16", "w8a8", "w4a8")[i % 3]
        step = 16 if fmt == "w8a8" else 128
        T = int(rng.integers(5, 200))
        H = step * int(rng.integers(1, 1536 // step + 1))
        I = step * int(rng.integers(2 if fmt == "w4a16" else 1, 768 // step + 1))
        E = int(rng.integers(1, 65))
        k = int(rng.integers(1, min(E, 8) + 1))
        out.append((f"{tag}{i}_{fmt}_t{T}_h{H}_i{I}_e{E}_k{k}", wid0 + i, T, H, I, E, k, fmt))
    return out


@pytest.mark.parametrize("case", _sweep_cases() + _sweep_cases(30, 3031, "wsweep", 900),
                         ids=lambda c: c[0])
def test_random_shapes_sweep(case):
    name, wid, T, H, I, E, k, fmt = case
    bias = "none" if fmt == "w8a8" else "normal"
    wl = synth.Workload(name, wid, T, H, I, E, k, fmt, bias, 1)
    if fmt == "w4a16":
        _w4_layer_case(wl, only_routed=False)
    elif fmt == "w8a8":
        _w8_case(wl)
    else:
        _w4a8_case(wl)


def test_empty_batch_all_entry_points():
    import quantized_moe_expert_top_amd as moe
    for fmt in ("w4a16", "w4a8", "w8a8"):
        b = moe.LayerBuffers.alloc(0, 256, 128, 8, 2, fmt)
        x = torch.empty((0, 256), dtype=torch.int16, device="cuda")
        L = torch.empty((0, 8), dtype=torch.float32, device="cuda")
        dummy = torch.empty(16, dtype=torch.uint8, device="cuda")
        moe.moe_forward(b, x, L, (dummy, dummy, dummy, dummy))
        torch.cuda.synchronize()
        assert np.all(to_np(b.offsets) == 0) and int(to_np(b.n_active)[0]) == 0
    # the whole-layer entry with no token: offsets all zero, no active expert
    b = moe.LayerBuffers.alloc(0, 256, 128, 8, 2, "w4a16")
    b.offsets.fill_(-1)
    b.n_active.fill_(-1)
    moe.moe_layer(b, x, L, (dummy, dummy, dummy, dummy))
    torch.cuda.synchronize()
    assert np.all(to_np(b.offsets) == 0) and int(to_np(b.n_active)[0]) == 0


# ------------------------------------------------------------ whole layer --
def _layer_entry(wl, x, L, weights):
    import quantized_moe_expert_top_amd as moe
    b = moe.LayerBuffers.alloc(wl.T, wl.H, wl.I, wl.E, wl.k, "w4a16")
    moe.moe_layer(b, to_dev(x), to_dev(L), weights)
    torch.cuda.synchronize()
    R = wl.T * wl.k
    n = int(to_np(b.n_active)[0])
    return {"ids": to_np(b.ids), "w": to_np(b.w), "expert_offsets": to_np(b.offsets),
            "sorted_slot": to_np(b.sorted_slot)[:R], "slot_pos": to_np(b.slot_pos)[:R],
            "n_active": n, "active": to_np(b.active)[:n],
            "y": to_np(b.y)[:R].astype(np.float64), "out": to_np(b.out).astype(np.float64),
            "y_bits": to_np(b.y)[:R].copy(), "out_bits": to_np(b.out).view(np.uint32).copy()}


LAYER_CASES = [
    # name, wid, T, H, I, E, k
    ("layer_t1", 301, 1, 256, 128, 8, 2),
    ("layer_t3_ragged", 302, 3, 384, 384, 16, 4),
    ("layer_t4_k32", 303, 4, 256, 256, 64, 32),     # R = 128: the largest fused batch
    ("layer_t4_e1024", 304, 4, 512, 256, 1024, 8),
    ("layer_t9_unfused", 305, 9, 256, 128, 8, 2),
]


@pytest.mark.parametrize("case", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_layer_entry_matches_oracle_and_calls(case):
    name, wid, T, H, I, E, k = case
    wl = synth.Workload(name, wid, T, H, I, E, k, "w4a16", "normal", 1)
    x, L = synth.x_bf16(wl, 0), synth.router_logits(wl, 0)
    ref = oracle.moe_layer_w4a16(x, L, wl.k, expert_getter_w4(wl, 0))
    wts = stage_weights(wl, 0)
    _say("layer entry", name, (T, H, I, E, k))
    got = _layer_entry(wl, x, L, wts)
    check_routing_and_perm(got, ref)
    assert_close(got["y"], ref["y"], "y")
    assert_close(got["out"], ref["out"], "out")
    calls = run_layer(wl, x, L, wts)
    np.testing.assert_array_equal(got["y_bits"], calls["y_bits"])
    np.testing.assert_array_equal(got["out_bits"], calls["out_bits"])


PREFILL_LAYER_CASES = [
    # name, wid, T, H, I, E, k, router bias
    ("lp_t512", 331, 512, 2048, 768, 128, 8, "normal"),   # the prompt shape: 4096 routed slots
    ("lp_t40_e1024", 332, 40, 256, 256, 1024, 8, "normal"),   # the largest E
    ("lp_t64_k32", 333, 64, 256, 256, 64, 32, "normal"),   # 2048 slots at k 32
    ("lp_t33_e1", 334, 33, 256, 256, 1, 1, "none"),        # every token on one expert
    ("lp_t520", 335, 520, 256, 256, 64, 8, "normal"),      # 4160 slots, ragged m-tiles
]
# (I >= 256: below it the bf16 rounding of h alone moves single y elements
# past 2% of the row rms, as at _sweep_cases)


@pytest.mark.parametrize("case", PREFILL_LAYER_CASES, ids=[c[0] for c in PREFILL_LAYER_CASES])
def test_layer_entry_prefill_matches_calls(case):
    """Prefill shapes (T > 4) through the whole-layer entry: routing,
    permutation, y and out are bit for bit those of the separate calls (route,
    permute, grouped FFN, combine); the smaller cases also against the
    oracle."""
    name, wid, T, H, I, E, k, bias = case
    wl = synth.Workload(name, wid, T, H, I, E, k, "w4a16", bias, 1)
    x, L = synth.x_bf16(wl, 0), synth.router_logits(wl, 0)
    wts = stage_weights(wl, 0)
    _say("prefill layer entry", name, (T, H, I, E, k))
    got = _layer_entry(wl, x, L, wts)
    calls = run_layer(wl, x, L, wts)
    for key in ("ids", "expert_offsets", "sorted_slot", "slot_pos", "active", "y_bits",
                "out_bits"):
        np.testing.assert_array_equal(got[key], calls[key], err_msg=key)
    assert got["n_active"] == calls["n_active"]
    if T * H <= 64 * 1024:
        ref = oracle.moe_layer_w4a16(x, L, wl.k, expert_getter_w4(wl, 0))
        check_routing_and_perm(got, ref)
        assert_close(got["y"], ref["y"], "y")
        assert_close(got["out"], ref["out"], "out")


def _layer_sweep_cases(n=10, seed=2027, tag="lsweep", wid0=420):
    """Seeded random decode shapes for the whole-layer entry (T <= 4, the fused
    kernels): H up to 3072 and I from 256 in steps of 128, E from 1 to 300,
    k up to min(E, 16); slot-per-block and persistent gate/up and every lane
    split they pick. I >= 256 for the reason given at _sweep_cases."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        T = int(rng.integers(1, 5))
        H = 128 * int(rng.integers(1, 25))
        I = 128 * int(rng.integers(2, 9))
        E = int(rng.integers(1, 301))
        k = int(rng.integers(1, min(E, 16) + 1))
        out.append((f"{tag}{i}_t{T}_h{H}_i{I}_e{E}_k{k}", wid0 + i, T, H, I, E, k))
    return out


@pytest.mark.parametrize("case", _layer_sweep_cases() + _layer_sweep_cases(20, 3033, "wlsweep", 940),
                         ids=lambda c: c[0])
def test_layer_entry_random_shapes(case):
    name, wid, T, H, I, E, k = case
    wl = synth.Workload(name, wid, T, H, I, E, k, "w4a16", "normal", 1)
    x, L = synth.x_bf16(wl, 0), synth.router_logits(wl, 0)
    ref = oracle.moe_layer_w4a16(x, L, wl.k, expert_getter_w4(wl, 0))
    _say("layer entry sweep", name)
    got = _layer_entry(wl, x, L, stage_weights(wl, 0, ref["perm"]["active"]))
    check_routing_and_perm(got, ref)
    assert_close(got["y"], ref["y"], "y")
    assert_close(got["out"], ref["out"], "out")


@pytest.mark.parametrize("name,unit", [("decode_t2", 0), ("decode_t2", 17), ("decode_large", 5),
                                       ("tiny", 0)])
def test_layer_entry_workloads(name, unit):
    wl = synth.workload(name)
    x, L = synth.x_bf16(wl, unit), synth.router_logits(wl, unit)
    ref = oracle.moe_layer_w4a16(x, L, wl.k, expert_getter_w4(wl, unit))
    wts = stage_weights(wl, unit, ref["perm"]["active"])
    _say("layer entry", name, unit)
    got = _layer_entry(wl, x, L, wts)
    check_routing_and_perm(got, ref)
    assert_close(got["out"], ref["out"], "out")
    again = _layer_entry(wl, x, L, wts)
    np.testing.assert_array_equal(got["out_bits"], again["out_bits"])


@pytest.mark.parametrize("case", [("layer_t4_h8192", 308, 4, 8192, 512, 32, 8),
                                  ("layer_t3_h8192", 308, 3, 8192, 512, 32, 8),
                                  ("layer_t4_h2048_k4", 328, 4, 2048, 768, 16, 4)],
                         ids=["t4_h8192", "t3_h8192", "t4_h2048_k4"])
def test_layer_entry_wide_tiles(case):
    """Fused layers with an expert that every token picked (3 or 4 rows: two
    row-pair passes), against the oracle; a second call gives the same bits.
    H 8192: the persistent gate/up (grid past the slot-per-block limit) and
    down tiles of several items per lane group (16 row pairs per block).
    H 2048, 16 routed slots: the slot-per-block gate/up with 32 lanes per
    unit."""
    name, wid, T, H, I, E, k = case
    wl = synth.Workload(name, wid, T, H, I, E, k, "w4a16", "normal", 1)
    x, L = synth.x_bf16(wl, 0), synth.router_logits(wl, 0)
    ref = oracle.moe_layer_w4a16(x, L, wl.k, expert_getter_w4(wl, 0))
    wts = stage_weights(wl, 0, ref["perm"]["active"])
    _say("layer entry", name, (T, H, I, E, k))
    got = _layer_entry(wl, x, L, wts)
    check_routing_and_perm(got, ref)
    assert np.diff(ref["perm"]["expert_offsets"]).max() == T   # an expert takes every token
    assert_close(got["y"], ref["y"], "y")
    assert_close(got["out"], ref["out"], "out")
    again = _layer_entry(wl, x, L, wts)
    np.testing.assert_array_equal(got["out_bits"], again["out_bits"])


def test_layer_entry_in_graph_replays():
    """The fused decode layer captured in a HIP graph: every replay matches the
    eager result (the layer keeps no state between calls: its second kernel
    takes the combine inside each block, with no counters)."""
    import quantized_moe_expert_top_amd as moe
    wl = synth.workload("decode_t2")
    units = [0, 1, 2]
    bufs, ins = [], []
    for u in units:
        x, L = synth.x_bf16(wl, u), synth.router_logits(wl, u)
        ins.append((to_dev(x), to_dev(L), stage_weights(wl, u)))
        bufs.append(moe.LayerBuffers.alloc(wl.T, wl.H, wl.I, wl.E, wl.k, "w4a16"))
    eager = []
    for b, (x, L, w) in zip(bufs, ins):
        moe.moe_layer(b, x, L, w)
    torch.cuda.synchronize()
    eager = [to_np(b.out).view(np.uint32).copy() for b in bufs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for b, (x, L, w) in zip(bufs, ins):
            moe.moe_layer(b, x, L, w)
    for rep in range(3):
        for b in bufs:
            b.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, b in enumerate(bufs):
            np.testing.assert_array_equal(to_np(b.out).view(np.uint32), eager[i])


def test_full_decode_step_graph_replays_match_eager():
    """The step bench.py times: all 48 layers of decode_t2 captured in one HIP
    graph; three replays (with eager work and synchronizations between them)
    match the eager pass bit for bit in every layer's out."""
    import quantized_moe_expert_top_amd as moe
    wl = synth.workload("decode_t2")
    bufs, ins = [], []
    for u in range(wl.units):
        x, L = synth.x_bf16(wl, u), synth.router_logits(wl, u)
        active = oracle.permute(oracle.route_topk(L, wl.k)[0], wl.E)["active"]
        ins.append((to_dev(x), to_dev(L), stage_weights(wl, u, active)))
        bufs.append(moe.LayerBuffers.alloc(wl.T, wl.H, wl.I, wl.E, wl.k, "w4a16"))
    _say("48-layer step graph", wl.name)
    for b, (x, L, w) in zip(bufs, ins):
        moe.moe_layer(b, x, L, w)
    torch.cuda.synchronize()
    eager = [to_np(b.out).view(np.uint32).copy() for b in bufs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for b, (x, L, w) in zip(bufs, ins):
            moe.moe_layer(b, x, L, w)
    for rep in range(3):
        for b in bufs:
            b.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for u, b in enumerate(bufs):
            np.testing.assert_array_equal(to_np(b.out).view(np.uint32), eager[u],
                                          err_msg=f"replay {rep}, layer {u}")


# ------------------------------------------------------- batch invariance --
INVARIANCE_CASES = [
    # T, tokens per sub-batch, path (layer entry: fused decode; calls: MFMA GEMM)
    (4, 1, "layer"),   # persistent gate/up for the batch, slot-per-block alone
    (4, 2, "layer"),
    (40, 20, "calls"),
    (512, 128, "calls"),   # the prompt shape on the MFMA GEMMs, against four batches of 128
    (512, 128, "layer"),   # the same through the layer entry
]


@pytest.mark.parametrize("case", INVARIANCE_CASES, ids=[f"t{c[0]}_{c[1]}_{c[2]}" for c in INVARIANCE_CASES])
def test_batch_invariance(case):
    """A token's layer output is bitwise the same whether it runs in a batch of
    T or in a smaller batch: per output element the kernels take the same
    arithmetic in the same order whatever else is in the batch."""
    T, sub, path = case
    wl = synth.Workload(f"inv_t{T}", 140 + T, T, 2048, 768, 128, 8, "w4a16", "normal", 1)
    x, L = synth.x_bf16(wl, 0), synth.router_logits(wl, 0)
    wts = stage_weights(wl, 0)
    run = _layer_entry if path == "layer" else run_layer
    _say("batch invariance", wl.name, T, sub, path)
    full = run(wl, x, L, wts)
    for t0 in range(0, T, sub):
        part = run(wl.with_(T=sub), x[t0:t0 + sub], L[t0:t0 + sub], wts)
        np.testing.assert_array_equal(part["out_bits"], full["out_bits"][t0:t0 + sub])



# ------------------------------------------------------ router projection --
ROUTER_CASES = [
    # name, wid, T, H, E
    ("router_decode", 401, 2, 2048, 128),
    ("router_t5_ragged", 406, 5, 192, 37),    # the few-token path with E % 4 != 0
    ("router_ragged", 402, 45, 192, 40),      # partial token and expert tiles
    ("router_prefill", 403, 512, 2048, 128),
    ("router_large", 404, 2, 7168, 256),
    ("router_e1024_few", 405, 7, 256, 1024),    # the few-token path at the largest E
    ("router_e1024", 407, 40, 256, 1024),       # the MFMA path at the largest E
]


@pytest.mark.parametrize("case", ROUTER_CASES, ids=[c[0] for c in ROUTER_CASES])
def test_router_logits_and_routing(case):
    """Logits within the float32 summation bound of the float64 oracle; the ids
    and weights routed from the GPU logits match the oracle's routing of those
    same logits (both sides decide on identical float32 inputs)."""
    import quantized_moe_expert_top_amd as moe
    name, wid, T, H, E = case
    wl = synth.Workload(name, wid, T, H, 128, E, 8, "w4a16", "none", 1)
    x, wr = synth.x_bf16(wl, 0), synth.router_weights(wl, 0)
    _say("router", name, T, H, E)
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    moe.router_logits(to_dev(x), to_dev(wr), logits)
    ids = torch.empty((T, 8), dtype=torch.int32, device="cuda")
    w = torch.empty((T, 8), dtype=torch.float32, device="cuda")
    moe.route_topk(logits, 8, ids, w)
    torch.cuda.synchronize()
    got = to_np(logits).astype(np.float64)
    ref = oracle.router_projection(x, wr)
    # float32 accumulation of H exact products: |err| <= H * 2^-24 * sum |x w|
    mag = np.abs(oracle.bf16_to_f64(x)) @ np.abs(oracle.bf16_to_f64(wr)).T
    assert np.all(np.abs(got - ref) <= H * 2.0 ** -24 * mag + 1e-30)
    rid, rw = oracle.route_topk(to_np(logits), 8)
    np.testing.assert_array_equal(to_np(ids), rid)
    np.testing.assert_allclose(to_np(w), rw, rtol=0, atol=1e-6)


def test_router_logits_deterministic():
    import quantized_moe_expert_top_amd as moe
    wl = synth.Workload("router_det", 405, 300, 1024, 128, 96, 8, "w4a16", "none", 1)
    x, wr = to_dev(synth.x_bf16(wl, 0)), to_dev(synth.router_weights(wl, 0))
    a = torch.empty((300, 96), dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    moe.router_logits(x, wr, a)
    moe.router_logits(x, wr, b)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(a).view(np.uint32), to_np(b).view(np.uint32))


# --------------------------------------------------------------- telemetry --
def test_expert_counts_accumulate_over_layers_and_steps():
    """Counts from the device permutation of several layers over four steps,
    one launch per step over a strided [L][E + 3] offsets array; the counters
    start above 2^32 so a 32-bit add would show."""
    import quantized_moe_expert_top_amd as moe
    E, L = 128, 3
    shapes = [(2, 8, 0.0), (512, 8, 1.1), (37, 4, 0.0)]
    base = np.int64(2 ** 33 - 5)
    want = np.full((L, E), base, np.int64)
    counts = torch.full((L, E), int(base), dtype=torch.int64, device="cuda")
    offs = torch.full((L, E + 3), -9, dtype=torch.int32, device="cuda")
    for step in range(4):
        for l, (T, k, skew) in enumerate(shapes):
            ids = _random_ids(T, E, k, seed=1000 * step + l, skew=skew)
            p = _permute_gpu(ids, E)
            offs[l, :E + 1] = to_dev(p["expert_offsets"].astype(np.int32))
            want[l] += oracle.expert_loads(ids, E)
        _say("expert counts step", step)
        moe.expert_counts_accumulate(offs, counts)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(counts), want)


def test_expert_counts_from_the_layer_entry():
    """The offsets moe_layer_w4a16 writes feed the counters directly."""
    import quantized_moe_expert_top_amd as moe
    wl = synth.workload("decode_t2")
    counts = torch.zeros(wl.E, dtype=torch.int64, device="cuda")
    want = np.zeros(wl.E, np.int64)
    for u in range(3):
        x, L = synth.x_bf16(wl, u), synth.router_logits(wl, u)
        b = moe.LayerBuffers.alloc(wl.T, wl.H, wl.I, wl.E, wl.k, "w4a16")
        ids, _ = oracle.route_topk(L, wl.k)
        wts = stage_weights(wl, u, np.unique(ids))
        moe.moe_layer(b, to_dev(x), to_dev(L), wts)
        moe.expert_counts_accumulate(b.offsets, counts)
        want += oracle.expert_loads(ids, wl.E)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(counts), want)


@pytest.mark.parametrize("E", [1, 8, 128, 256, 1024])
def test_expert_hot_rank_matches_oracle(E):
    """Many ties (a small value range) in both 32-bit halves of the counts."""
    import quantized_moe_expert_top_amd as moe
    rng = np.random.default_rng(E)
    L = 3
    c = (rng.integers(0, 3, size=(L, E)).astype(np.uint64) << np.uint64(32)) + \
        rng.integers(0, 4, size=(L, E)).astype(np.uint64)
    counts = to_dev(c.view(np.int64))
    for n in sorted({1, max(E // 2, 1), E}):
        hot = torch.full((L, n), -5, dtype=torch.int32, device="cuda")
        _say("hot rank", E, n)
        moe.expert_hot_rank(counts, n, hot)
        torch.cuda.synchronize()
        got = to_np(hot)
        for l in range(L):
            np.testing.assert_array_equal(got[l], oracle.hot_rank(c[l], n))
