"""Pins of the CPU oracle to things other than itself: hand-worked fixtures
(tests/golden/), closed forms, brute force on tiny inputs, invariants, and
independent library routines. The last section plants mistakes into copies of
oracle functions and shows that a pin catches each one."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- dequant --
def _dequant_case():
    d = gold("dequant_hand.json")
    row = np.full(d["K"] // 2, d["bytes_default"], np.uint8)
    for i, b in d["bytes_set"].items():
        row[int(i)] = b
    return d, row[None, :], np.array([d["scale_bits"]], np.uint16)


def expected_dequant(d):
    want = np.zeros(d["K"])
    for i, v in d["expected_nonzero"].items():
        want[int(i)] = v
    return want


def test_fp16_scale_decode_golden():
    d = gold("dequant_hand.json")
    np.testing.assert_array_equal(oracle.fp16_to_f64(np.array(d["scale_bits"], np.uint16)), d["scale_values"])
    assert oracle.fp16_to_f64(np.array([d["subnormal_scale_bits"]], np.uint16))[0] == d["subnormal_scale_value"]


def test_dequant_golden_nibble_order_and_group_boundary():
    d, packed, sc = _dequant_case()
    w = oracle.dequant_w4(packed, sc)[0]
    np.testing.assert_array_equal(w, expected_dequant(d))


def test_dequant_subnormal_scale_kept():
    d = gold("dequant_hand.json")
    packed = np.full((1, 64), 0xFF, np.uint8)
    sc = np.array([[d["subnormal_scale_bits"]]], np.uint16)
    w = oracle.dequant_w4(packed, sc)
    assert np.all(w == d["subnormal_code15_value"])


@pytest.mark.parametrize("code,mult", [(8, 0.0), (0, -8.0), (15, 7.0)])
def test_dequant_special_codes(code, mult):
    s = np.float16(0.013671875)   # exact in fp16
    packed = np.full((3, 128), code | (code << 4), np.uint8)
    sc = np.full((3, 2), s.view(np.uint16), np.uint16)
    w = oracle.dequant_w4(packed, sc)
    assert np.all(w == mult * float(s))


def test_dequant_round_trip():
    rng = np.random.default_rng(11)
    q = rng.integers(0, 16, size=(5, 256))
    s = (0.02 * np.abs(rng.standard_normal((5, 2))) + 1e-3).astype(np.float16)
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    w = oracle.dequant_w4(packed, s.view(np.uint16))
    sf = np.repeat(s.astype(np.float64), 128, axis=1)
    q_back = np.rint(w / sf) + 8
    np.testing.assert_array_equal(q_back, q)
    np.testing.assert_array_equal((q_back - 8) * sf, w)


def test_unpack_against_bit_loop():
    rng = np.random.default_rng(3)
    packed = rng.integers(0, 256, size=(4, 32), dtype=np.uint8)
    q = oracle.unpack_int4(packed)
    for n in range(4):
        for kk in range(64):
            byte = int(packed[n, kk // 2])
            want = (byte >> (4 * (kk % 2))) & 0xF
            assert q[n, kk] == want


# ----------------------------------------------------------------- routing --
def test_route_golden():
    for c in gold("route_hand.json")["cases"]:
        L = np.array(c["logits"], np.float32)
        ids, w = oracle.route_topk(L, c["k"])
        np.testing.assert_array_equal(ids, c["ids"])
        np.testing.assert_allclose(w, c["w"], rtol=0, atol=1e-15)


def _brute_topk(row, k):
    return sorted(range(len(row)), key=lambda e: (-float(row[e]), e))[:k]


@pytest.mark.parametrize("E,k", [(8, 2), (16, 5), (64, 8), (128, 8), (7, 7)])
def test_route_bruteforce_with_ties(E, k):
    rng = np.random.default_rng(E * 31 + k)
    # small integer range forces many ties; sign-flipped zeros mixed in
    L = rng.integers(-3, 4, size=(40, E)).astype(np.float32)
    L[L == 0] = np.where(rng.random(np.count_nonzero(L == 0)) < 0.5, 0.0, -0.0)
    ids, w = oracle.route_topk(L, k)
    for t in range(L.shape[0]):
        assert list(ids[t]) == _brute_topk(L[t], k)
        sel = [float(L[t, e]) for e in ids[t]]
        z = [math.exp(v - sel[0]) for v in sel]
        np.testing.assert_allclose(w[t], [v / sum(z) for v in z], rtol=1e-14)


def test_route_k1_is_first_argmax():
    rng = np.random.default_rng(5)
    L = rng.integers(-2, 3, size=(100, 9)).astype(np.float32)
    ids, w = oracle.route_topk(L, 1)
    np.testing.assert_array_equal(ids[:, 0], np.argmax(L, axis=1))
    assert np.all(w == 1.0)


def test_route_k_equals_E_full_order_and_weights_sum():
    rng = np.random.default_rng(6)
    L = rng.standard_normal((20, 12)).astype(np.float32)
    ids, w = oracle.route_topk(L, 12)
    for t in range(20):
        assert sorted(ids[t]) == list(range(12))
        assert np.all(np.diff(L[t, ids[t]]) <= 0)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-15)
    # softmax over all E equals softmax over the k=E selection
    z = np.exp(L.astype(np.float64) - L.max(1, keepdims=True))
    full = z / z.sum(1, keepdims=True)
    np.testing.assert_allclose(w, np.take_along_axis(full, ids.astype(np.int64), 1), rtol=1e-13)


def test_route_two_pick_closed_form():
    rng = np.random.default_rng(7)
    L = rng.standard_normal((50, 6)).astype(np.float32)
    ids, w = oracle.route_topk(L, 2)
    l0 = L[np.arange(50), ids[:, 0]].astype(np.float64)
    l1 = L[np.arange(50), ids[:, 1]].astype(np.float64)
    np.testing.assert_allclose(w[:, 0], 1.0 / (1.0 + np.exp(l1 - l0)), rtol=1e-14)


# ------------------------------------------------------------- permutation --
def _check_perm_invariants(ids, E, p):
    T, k = ids.shape
    R = T * k
    off = p["expert_offsets"].astype(np.int64)
    ss = p["sorted_slot"].astype(np.int64)
    sp = p["slot_pos"].astype(np.int64)
    counts = np.array([np.count_nonzero(ids == e) for e in range(E)])
    assert off[0] == 0 and off[-1] == R
    np.testing.assert_array_equal(np.diff(off), counts)
    assert sorted(ss.tolist()) == list(range(R))
    np.testing.assert_array_equal(sp[ss], np.arange(R))
    flat = ids.reshape(-1)
    for e in range(E):
        blk = ss[off[e]:off[e + 1]]
        assert np.all(flat[blk] == e)
        assert np.all(np.diff(blk) > 0)
    tok_hits = np.bincount(ss // k, minlength=T)
    assert np.all(tok_hits == k)
    np.testing.assert_array_equal(p["active"], [e for e in range(E) if counts[e] > 0])
    assert p["n_active"] == int((counts > 0).sum())


@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (2, 128, 8), (37, 20, 3), (300, 128, 8), (1, 4, 4)])
def test_permute_invariants(T, E, k):
    rng = np.random.default_rng(T + E + k)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    p = oracle.permute(ids, E)
    _check_perm_invariants(ids, E, p)


def test_permute_bruteforce():
    rng = np.random.default_rng(9)
    T, E, k = 25, 6, 3
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    p = oracle.permute(ids, E)
    order = []
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if ids[t, j] == e:
                    order.append(t * k + j)
    np.testing.assert_array_equal(p["sorted_slot"], order)


# --------------------------------------------------------------------- FFN --
def test_ffn_hand_closed_form():
    d = gold("ffn_hand.json")
    H, I = d["H"], d["I"]
    x = np.full((1, H), d["x_bf16_bits"], np.uint16)
    w13 = np.empty((2 * I, H // 2), np.uint8)
    w13[:I] = d["gate_byte"]
    w13[I:] = d["up_byte"]
    s13 = np.full((2 * I, H // 128), d["scale_bits"], np.uint16)
    w2 = np.full((H, I // 2), d["w2_byte"], np.uint8)
    s2 = np.full((H, I // 128), d["scale_bits"], np.uint16)
    r = oracle.moe_layer_w4a16(x, np.zeros((1, 1), np.float32), 1, lambda e: (w13, s13, w2, s2))
    np.testing.assert_allclose(r["out"], d["out_value"], rtol=1e-15)
    assert d["out_value"] == 2.0 / (1.0 + math.exp(-1.0))


def _tiny(name="tiny"):
    wl = synth.workload(name)
    x = synth.x_bf16(wl, 0)
    L = synth.router_logits(wl, 0)
    get = lambda e: synth.expert_w4(wl, 0, e, "w13") + synth.expert_w4(wl, 0, e, "w2")  # noqa: E731
    return wl, x, L, get


def test_ffn_bruteforce_per_token_matches_grouped():
    """Per token, loop over its k experts with no permutation and sum directly."""
    wl, x, L, get = _tiny()
    r = oracle.moe_layer_w4a16(x, L, wl.k, get)
    X = oracle.bf16_to_f64(x)
    out = np.zeros((wl.T, wl.H))
    for t in range(wl.T):
        for j in range(wl.k):
            w13, s13, w2, s2 = get(int(r["ids"][t, j]))
            W13 = oracle.dequant_w4(w13, s13)
            W2 = oracle.dequant_w4(w2, s2)
            g = np.array([np.dot(W13[n], X[t]) for n in range(wl.I)])
            u = np.array([np.dot(W13[wl.I + n], X[t]) for n in range(wl.I)])
            h = g * (1.0 + np.tanh(g / 2.0)) / 2.0 * u      # silu via the tanh identity
            y = np.array([np.dot(W2[m], h) for m in range(wl.H)])
            out[t] += r["w"][t, j] * y
    np.testing.assert_allclose(r["out"], out, rtol=1e-11, atol=1e-11)


def test_e1_k1_reduces_to_dense_ffn():
    rng = np.random.default_rng(21)
    H, I, T = 256, 128, 5
    xb = synth.bf16_bits_from_f32(rng.standard_normal((T, H)).astype(np.float32))
    w13 = rng.integers(0, 256, size=(2 * I, H // 2), dtype=np.uint8)
    s13 = (0.02 * np.abs(rng.standard_normal((2 * I, H // 128)))).astype(np.float16).view(np.uint16)
    w2 = rng.integers(0, 256, size=(H, I // 2), dtype=np.uint8)
    s2 = (0.02 * np.abs(rng.standard_normal((H, I // 128)))).astype(np.float16).view(np.uint16)
    r = oracle.moe_layer_w4a16(xb, rng.standard_normal((T, 1)).astype(np.float32), 1,
                               lambda e: (w13, s13, w2, s2))
    assert np.all(r["w"] == 1.0)
    X = oracle.bf16_to_f64(xb)
    Wg = oracle.dequant_w4(w13, s13)[:I]
    Wu = oracle.dequant_w4(w13, s13)[I:]
    W2 = oracle.dequant_w4(w2, s2)
    G = np.einsum("ti,ni->tn", X, Wg)
    U = np.einsum("ti,ni->tn", X, Wu)
    dense = np.einsum("tn,hn->th", G * 0.5 * (1 + np.tanh(0.5 * G)) * U, W2)
    np.testing.assert_allclose(r["out"], dense, rtol=1e-11, atol=1e-11)


def test_zero_down_codes_and_zero_x_give_exact_zero():
    wl, x, L, get = _tiny()

    def get_w2_zero(e):
        w13, s13, w2, s2 = get(e)
        return w13, s13, np.full_like(w2, 0x88), s2
    r = oracle.moe_layer_w4a16(x, L, wl.k, get_w2_zero)
    assert np.all(r["out"] == 0.0)
    r = oracle.moe_layer_w4a16(np.zeros_like(x), L, wl.k, get)
    assert np.all(r["out"] == 0.0)


def test_combine_order_golden():
    d = gold("combine_order.json")
    Y = np.array(d["y_rows"])
    w = np.array(d["w"])
    out = oracle.combine(Y, np.arange(3), w)
    np.testing.assert_array_equal(out, d["out"])


# -------------------------------------------------------------------- W8A8 --
def test_quant_rows_golden():
    for c in gold("quant_hand.json")["cases"]:
        q, s = oracle.quant_rows_int8(np.array([c["x"]], np.float32))
        assert float(s[0]) == c["s"]
        np.testing.assert_array_equal(q[0], c["q"])


def test_quant_rows_bounds_and_scale_rule():
    rng = np.random.default_rng(4)
    a = (rng.standard_normal((64, 300)) * rng.uniform(0.01, 100, (64, 1))).astype(np.float32)
    q, s = oracle.quant_rows_int8(a)
    assert q.dtype == np.int8 and np.all(np.abs(q.astype(int)) <= 127)
    np.testing.assert_array_equal(s, (np.abs(a).max(1) / np.float32(127)).astype(np.float32))
    # the absmax element maps to +-127 and every code is within half a step
    assert np.all(np.abs(q).max(1) == 127)
    err = np.abs(a / s[:, None] - q)
    assert np.all(err <= 0.5 + 1e-4)


def test_int_matmul_exact_against_integer_matmul():
    rng = np.random.default_rng(8)
    A = rng.integers(-127, 128, size=(17, 2048), dtype=np.int8)
    B = rng.integers(-127, 128, size=(33, 2048), dtype=np.int8)
    np.testing.assert_array_equal(oracle.int_matmul_exact(A, B),
                                  np.matmul(A.astype(np.int64), B.astype(np.int64).T))
    A = np.full((2, 2048), 127, np.int8)
    B = np.full((3, 2048), -127, np.int8)
    assert np.all(oracle.int_matmul_exact(A, B) == -2048 * 127 * 127)


def _w8_small(seed=0, T=12, H=256, I=128, E=6, k=2):
    wl = synth.Workload("w8_small", 90 + seed, T, H, I, E, k, "w8a8", "none", 1)
    x = synth.x_bf16(wl, 0)
    L = synth.router_logits(wl, 0)
    get = lambda e: synth.expert_w8(wl, 0, e, "w13") + synth.expert_w8(wl, 0, e, "w2")  # noqa: E731
    return wl, x, L, get


def test_w8a8_bruteforce_per_token():
    """Each routed slot recomputed on its own with explicit integer loops."""
    wl, x, L, get = _w8_small()
    r = oracle.moe_layer_w8a8(x, L, wl.k, get)
    X = oracle.bf16_to_f64(x).astype(np.float32)
    out = np.zeros((wl.T, wl.H))
    for t in range(wl.T):
        xq, xs = oracle.quant_rows_int8(X[t:t + 1])
        for j in range(wl.k):
            e = int(r["ids"][t, j])
            w13, s13, w2, s2 = get(e)
            acc = w13.astype(np.int64) @ xq[0].astype(np.int64)
            p = r["perm"]["slot_pos"][t * wl.k + j]
            np.testing.assert_array_equal(r["acc13"][p], acc)
            gu = acc * float(xs[0]) * s13.astype(np.float64)
            h = gu[:wl.I] * 0.5 * (1 + np.tanh(0.5 * gu[:wl.I])) * gu[wl.I:]
            hq, hs = oracle.quant_rows_int8(h[None].astype(np.float32))
            acc2 = w2.astype(np.int64) @ hq[0].astype(np.int64)
            np.testing.assert_array_equal(r["acc2"][p], acc2)
            out[t] += r["w"][t, j] * acc2 * float(hs[0]) * s2.astype(np.float64)
    np.testing.assert_allclose(r["out"], out, rtol=1e-12, atol=1e-12)


def test_w8a8_close_to_unquantized_activations():
    """Quantizing activations is the only approximation on top of the int8
    weights: the result stays within a few percent of the float64 FFN on
    dequantized int8 weights (a loose sanity bound, 127 levels per row)."""
    wl, x, L, get = _w8_small(seed=1, T=32)
    r = oracle.moe_layer_w8a8(x, L, wl.k, get)
    X = oracle.bf16_to_f64(x)
    ref = np.zeros((wl.T, wl.H))
    for t in range(wl.T):
        for j in range(wl.k):
            w13, s13, w2, s2 = get(int(r["ids"][t, j]))
            y = oracle.expert_ffn(X[t:t + 1], w13 * s13[:, None].astype(np.float64),
                                  w2 * s2[:, None].astype(np.float64))[0]
            ref[t] += r["w"][t, j] * y
    rel = np.linalg.norm(r["out"] - ref) / np.linalg.norm(ref)
    assert rel < 0.03


# ---------------------------------------------------------- real workloads --
@pytest.mark.parametrize("name", ["tiny", "decode_t2"])
def test_workload_routing_invariants(name):
    wl = synth.workload(name)
    L = synth.router_logits(wl, 0)
    ids, w = oracle.route_topk(L, wl.k)
    p = oracle.permute(ids, wl.E)
    _check_perm_invariants(ids, wl.E, p)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-14)


# --------------------------------------------------- planted mistakes (CPU) --
def _swapped_nibbles(packed, scale_bits):
    p = np.asarray(packed, np.uint8)
    q = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
    q[..., 0::2] = p >> 4          # planted: high nibble taken as even k
    q[..., 1::2] = p & 0x0F
    return (q.astype(np.float64) - 8) * np.repeat(oracle.fp16_to_f64(scale_bits), 128, axis=-1)


def _group_off_by_one(packed, scale_bits):
    q = oracle.unpack_int4(packed).astype(np.float64)
    s = oracle.fp16_to_f64(scale_bits)
    idx = np.minimum((np.arange(q.shape[-1]) + 1) // 128, s.shape[-1] - 1)   # planted
    return (q - 8) * s[..., idx]


@pytest.mark.parametrize("bad", [_swapped_nibbles, _group_off_by_one])
def test_planted_dequant_mistakes_are_caught(bad):
    d, packed, sc = _dequant_case()
    assert not np.array_equal(bad(packed, sc)[0], expected_dequant(d))


def _route_high_index_ties(logits, k):
    L = np.asarray(logits, np.float32)
    E = L.shape[1]
    rev = np.argsort(-L[:, ::-1].astype(np.float64), axis=1, kind="stable")[:, :k]
    return (E - 1 - rev).astype(np.int32)   # planted: ties go to the higher index


def test_planted_tie_break_is_caught():
    caught = False
    for c in gold("route_hand.json")["cases"]:
        ids = _route_high_index_ties(np.array(c["logits"], np.float32), c["k"])
        caught |= not np.array_equal(ids, c["ids"])
    assert caught


def test_planted_unstable_permutation_is_caught():
    rng = np.random.default_rng(2)
    ids = np.stack([rng.choice(8, 2, replace=False) for _ in range(16)]).astype(np.int32)
    p = oracle.permute(ids, 8)
    bad = dict(p)
    ss = p["sorted_slot"].copy()
    off = p["expert_offsets"]
    e = int(np.argmax(np.diff(off)))
    ss[off[e]:off[e + 1]] = ss[off[e]:off[e + 1]][::-1]    # planted: reversed block
    bad["sorted_slot"] = ss
    with pytest.raises(AssertionError):
        _check_perm_invariants(ids, 8, bad)


def test_planted_reverse_combine_is_caught():
    d = gold("combine_order.json")
    Y = np.array(d["y_rows"])
    w = np.array(d["w"])
    out = np.zeros((1, 1))
    for j in reversed(range(3)):        # planted: reversed accumulation order
        out += w[:, j:j + 1] * Y[j]
    assert not np.array_equal(out, d["out"])


def test_planted_half_away_rounding_is_caught():
    c = gold("quant_hand.json")["cases"][0]
    x = np.array(c["x"], np.float32)
    s = np.float32(np.abs(x).max()) / np.float32(127)
    q_bad = np.sign(x / s) * np.floor(np.abs(x / s) + 0.5)   # planted: half away from zero
    assert not np.array_equal(q_bad, c["q"])


def test_planted_swapped_gate_up_is_caught():
    d = gold("ffn_hand.json")
    H, I = d["H"], d["I"]
    x = oracle.bf16_to_f64(np.full((1, H), d["x_bf16_bits"], np.uint16))
    w13 = np.empty((2 * I, H // 2), np.uint8)
    w13[:I] = d["gate_byte"]
    w13[I:] = d["up_byte"]
    W13 = oracle.dequant_w4(w13, np.full((2 * I, H // 128), d["scale_bits"], np.uint16))
    W2 = oracle.dequant_w4(np.full((H, I // 2), d["w2_byte"], np.uint8),
                           np.full((H, I // 128), d["scale_bits"], np.uint16))
    G, U = x @ W13[I:].T, x @ W13[:I].T          # planted: halves swapped
    bad = (oracle.silu(G) * U) @ W2.T
    assert not np.allclose(bad, d["out_value"], rtol=1e-6)


# ------------------------------------------------------ router projection --
def _bits(a):
    return synth.bf16_bits_from_f32(np.asarray(a, np.float32))


def test_router_projection_one_hot_rows_pick_router_columns():
    """x = e_h (an exact bf16 one) selects column h of the router rows exactly."""
    rng = np.random.default_rng(7)
    E, H = 5, 16
    wr = _bits(rng.standard_normal((E, H)))
    x = np.zeros((H, H), np.float32)
    x[np.arange(H), np.arange(H)] = 1.0
    got = oracle.router_projection(_bits(x), wr)
    np.testing.assert_array_equal(got, oracle.bf16_to_f64(wr).T)


def test_router_projection_closed_forms():
    # all ones: every logit is H; a row of twos against a row of 0.5: H
    H = 256
    ones = _bits(np.ones((2, H)))
    np.testing.assert_array_equal(oracle.router_projection(ones, _bits(np.ones((3, H)))),
                                  np.full((2, 3), float(H)))
    np.testing.assert_array_equal(
        oracle.router_projection(_bits(np.full((1, H), 2.0)), _bits(np.full((1, H), 0.5))),
        [[float(H)]])


def test_router_projection_against_fsum_loop():
    """Brute force: a Python loop with exactly rounded sums on tiny shapes."""
    rng = np.random.default_rng(11)
    T, H, E = 3, 24, 5
    xb, wb = _bits(rng.standard_normal((T, H))), _bits(rng.standard_normal((E, H)))
    xv, wv = oracle.bf16_to_f64(xb), oracle.bf16_to_f64(wb)
    want = np.array([[math.fsum(xv[t, h] * wv[e, h] for h in range(H)) for e in range(E)]
                     for t in range(T)])
    np.testing.assert_allclose(oracle.router_projection(xb, wb), want, rtol=0, atol=1e-12)


def test_planted_transposed_router_is_caught():
    """A copy that multiplies by the router rows untransposed (w_r treated as
    [H][E]) fails the one-hot pin on a square shape."""
    rng = np.random.default_rng(3)
    H = 8
    wr = _bits(rng.standard_normal((H, H)))
    x = np.eye(H, dtype=np.float32)

    def bad(x_bits, wr_bits):
        return oracle.bf16_to_f64(x_bits) @ oracle.bf16_to_f64(wr_bits)

    assert not np.array_equal(bad(_bits(x), wr), oracle.bf16_to_f64(wr).T)
    np.testing.assert_array_equal(oracle.router_projection(_bits(x), wr), oracle.bf16_to_f64(wr).T)


# ------------------------------------------------------------------- W4A8 --
def _w4a8_small(seed=0, T=10, H=256, I=128, E=6, k=2):
    wl = synth.Workload("w4a8_small", 95 + seed, T, H, I, E, k, "w4a8", "none", 1)
    x = synth.x_bf16(wl, 0)
    L = synth.router_logits(wl, 0)
    get = lambda e: synth.expert_w4(wl, 0, e, "w13") + synth.expert_w4(wl, 0, e, "w2")  # noqa: E731
    return wl, x, L, get


def _w4a8_slot_bruteforce(x_row, w13, s13, w2, s2, I):
    """One routed slot with explicit per-group int64 dot products (R9)."""
    xq, xs = oracle.quant_rows_int8(x_row[None].astype(np.float32))
    q13 = oracle.unpack_int4(w13).astype(np.int64) - 8
    sc13 = oracle.fp16_to_f64(s13)
    H = q13.shape[1]
    gu = np.zeros(2 * I)
    for n in range(2 * I):
        tot = 0.0
        for g in range(H // 128):
            d = int(np.dot(xq[0, g * 128:(g + 1) * 128].astype(np.int64), q13[n, g * 128:(g + 1) * 128]))
            tot += sc13[n, g] * d
        gu[n] = tot * float(xs[0])
    h = gu[:I] / (1.0 + np.exp(-gu[:I])) * gu[I:]
    hq, hs = oracle.quant_rows_int8(h[None].astype(np.float32))
    q2 = oracle.unpack_int4(w2).astype(np.int64) - 8
    sc2 = oracle.fp16_to_f64(s2)
    y = np.zeros(q2.shape[0])
    for n in range(q2.shape[0]):
        tot = 0.0
        for g in range(I // 128):
            d = int(np.dot(hq[0, g * 128:(g + 1) * 128].astype(np.int64), q2[n, g * 128:(g + 1) * 128]))
            tot += sc2[n, g] * d
        y[n] = tot * float(hs[0])
    return y


def test_w4a8_bruteforce_per_token():
    wl, x, L, get = _w4a8_small()
    r = oracle.moe_layer_w4a8(x, L, wl.k, get)
    X = oracle.bf16_to_f64(x)
    out = np.zeros((wl.T, wl.H))
    for t in range(wl.T):
        for j in range(wl.k):
            e = int(r["ids"][t, j])
            y = _w4a8_slot_bruteforce(X[t], *get(e), wl.I)
            np.testing.assert_allclose(r["y"][r["perm"]["slot_pos"][t * wl.k + j]], y,
                                       rtol=1e-12, atol=1e-12)
            out[t] += r["w"][t, j] * y
    np.testing.assert_allclose(r["out"], out, rtol=1e-12, atol=1e-12)


def test_w4a8_close_to_w4a16():
    """Same weights; only the activation quantization differs."""
    wl, x, L, get = _w4a8_small(seed=1, T=16)
    a = oracle.moe_layer_w4a8(x, L, wl.k, get)["out"]
    b = oracle.moe_layer_w4a16(x, L, wl.k, get)["out"]
    assert np.linalg.norm(a - b) / np.linalg.norm(b) < 3e-2


def test_w4a8_zero_down_codes_give_exact_zero():
    wl, x, L, get = _w4a8_small(seed=2)

    def zero_w2(e):
        w13, s13, w2, s2 = get(e)
        return w13, s13, np.full_like(w2, 0x88), s2

    assert np.all(oracle.moe_layer_w4a8(x, L, wl.k, zero_w2)["out"] == 0.0)


def test_planted_w4a8_zero_point_sign_is_caught():
    """A copy that adds the zero point instead of subtracting it fails the
    brute force."""
    wl, x, L, get = _w4a8_small(seed=3, T=4)

    def bad_get(e):
        w13, s13, w2, s2 = get(e)
        # codes q -> 16 - q (mod 16) flips q - 8 into 8 - q for every code but 8
        flip = lambda p: (((16 - (p & 15)) & 15) | (((16 - (p >> 4)) & 15) << 4)).astype(np.uint8)  # noqa: E731
        return flip(w13), s13, flip(w2), s2

    r = oracle.moe_layer_w4a8(x, L, wl.k, bad_get)
    X = oracle.bf16_to_f64(x)
    e = int(r["ids"][0, 0])
    y = _w4a8_slot_bruteforce(X[0], *get(e), wl.I)
    assert not np.allclose(r["y"][r["perm"]["slot_pos"][0]], y, rtol=1e-6)


# --------------------------------------------------------------- telemetry --
def test_expert_loads_and_hot_rank_hand_fixture():
    d = gold("hot_rank_hand.json")
    loads = oracle.expert_loads(np.array(d["ids"]), d["E"])
    assert loads.tolist() == d["loads"]
    assert oracle.hot_rank(loads, d["E"]).tolist() == d["hot_all"]
    assert oracle.hot_rank(loads, 3).tolist() == d["hot_all"][:3]
    assert oracle.hot_rank(loads, 0).tolist() == []


def test_expert_loads_match_permutation_blocks_and_total():
    """The loads are the lengths of the expert blocks of the stable
    permutation, and they add up to T * k (every routed row counted once)."""
    rng = np.random.default_rng(11)
    for T, E, k in ((1, 4, 1), (37, 16, 3), (300, 128, 8)):
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
        loads = oracle.expert_loads(ids, E)
        assert int(loads.sum()) == T * k
        off = oracle.permute(ids, E)["expert_offsets"]
        assert np.array_equal(loads, np.asarray(off[1:]) - np.asarray(off[:-1]))


def test_hot_rank_against_repeated_argmax():
    """A different algorithm: repeatedly take the first maximum and remove it
    (numpy argmax returns the first, i.e. lowest-index, maximum)."""
    rng = np.random.default_rng(12)
    for E in (1, 7, 64, 300):
        loads = rng.integers(0, 5, size=E)          # a small range: many ties
        left = loads.astype(np.int64).copy()
        want = []
        for _ in range(E):
            e = int(np.argmax(left))
            want.append(e)
            left[e] = -1
        for n in (0, 1, E // 2, E):
            assert oracle.hot_rank(loads, n).tolist() == want[:n]


def test_planted_hot_rank_tie_order_is_caught():
    """A copy that breaks ties toward the higher index fails the fixture."""
    d = gold("hot_rank_hand.json")
    loads = np.array(d["loads"])
    bad = sorted(range(len(loads)), key=lambda e: (-int(loads[e]), -e))
    assert bad != d["hot_all"]
