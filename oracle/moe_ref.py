"""CPU oracle for the routed mixture-of-experts FFN layer over group-quantized
expert weights.

TEST INFRASTRUCTURE ONLY. This module is the plain, slow reference the HIP path
is checked against. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product path
(``quantized_moe_expert_top_amd``) never does, and it shares no code with it
(its own nibble unpacker, its own bf16/fp16 decoding, its own routing).

Precision: float64 throughout, except where the method itself fixes float32
(the W8A8 dynamic quantization, whose codes are decided in float32 exactly as
the kernels decide them). Integer results (top-k ids, the permutation, the W8A8
int32 accumulators) are exact.

Sources. The three pages never write the layer's formulas down; they give its
shape and its checks:
  * "Performance and verification", section "Why it is fast": a prompt batch
    reads every routed expert it calls once (tokens grouped by expert); host
    experts go out as grouped dispatches, dot products taken on the quantized
    weights as stored; routed experts of a prompt run as grouped int8 GEMMs.
  * "Performance and verification", section "How it is verified": router ids
    and other integer outputs must match exactly; float outputs stay inside
    rounding-derived bands; an f64 copy serves as the reference.
  * "Measured results" (header and "Speed"): the W4A16 g128 weight format and
    the W4A8/W4A16 paths.
Everything else is the workload definition's reading of those words, listed
where each function states it:
  R1 top-k order: descending logit, ties to the lower expert index (+0 == -0).
  R2 router weights: softmax over the k selected logits only.
  R3 expert rows: a stable expert-contiguous order of the flat slots f = t*k+j.
  R4 int4 layout: [N][K/2] bytes, low nibble = even k; implicit zero point 8;
     one fp16 scale per (row n, 128-wide K group); W = (q - 8) * s.
  R5 W13 rows [0, I) are the gate projection, rows [I, 2I) the up projection;
     SwiGLU h = silu(gate) * up with silu(g) = g / (1 + exp(-g)).
  R6 combine: out[t] = sum_j w[t,j] * y[t,j], summed in increasing j.
  R7 W8A8: per-row absmax scale s = absmax/127 in float32 (s = 0 for a zero
     row), codes rint_half_even(x/s) clamped to [-127, 127]; the same rule for
     the activations x (one row per token) and for h (one row per routed slot);
     int8 x int8 -> exact integer accumulators; y = acc * s_row * s_channel.
  R9 W4A8: the int4 g128 weights of R4 against per-token int8 activations
     (the R7 rule): per 128-wide K group an exact integer dot product of the
     activation codes with (q - 8), times the group's fp16 scale, summed over
     groups, times the row's activation scale; SwiGLU; h re-quantized per
     routed row by R7; the down projection the same way.
  R8 router projection ahead of the top-k: logits[t, e] = sum_h x[t, h] *
     w_r[e, h] over the bf16 token rows and the bf16 router rows [E][H] (the
     pages route on such logits; the workload hands them in, and the step that
     makes them is the dense product of the two).
  R10 expert-load telemetry ("Performance and verification", section "Why it
     is fast": the engines count their own routing as they run and move the
     experts used most): a layer's per-expert load is the number of routed
     rows each expert received; loads add up over calls; the hot list of a
     layer is its experts by descending load, ties to the lower expert index.
"""
from __future__ import annotations

import numpy as np

GROUP = 128
ZERO_POINT = 8


# ---------------------------------------------------------------- decoding --
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact: bf16 is the top half of a float32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def fp16_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE half bit patterns -> float64 (exact, subnormals kept)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """[N, K/2] bytes -> [N, K] codes 0..15; byte i holds k=2i (low nibble)
    and k=2i+1 (high nibble) (reading R4)."""
    p = np.asarray(packed, dtype=np.uint8)
    q = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    q[..., 0::2] = p & 0x0F
    q[..., 1::2] = p >> 4
    return q


def dequant_w4(packed: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """W[n, k] = (q[n, k] - 8) * s[n, k // 128] in float64 (reading R4; the g128
    format of "Measured results")."""
    q = unpack_int4(packed).astype(np.float64)
    s = fp16_to_f64(scale_bits)
    return (q - ZERO_POINT) * np.repeat(s, GROUP, axis=-1)


# ----------------------------------------------------------------- routing --
def route_topk(logits: np.ndarray, k: int):
    """Per token: the k largest logits, descending, ties to the lower expert
    index (R1); weights = softmax over those k logits in float64 (R2).
    Exact integer ids are what "How it is verified" asks of router outputs."""
    L = np.asarray(logits, dtype=np.float32)
    assert L.ndim == 2 and np.isfinite(L).all(), "logits must be finite [T, E]"
    T, E = L.shape
    assert 1 <= k <= E
    # A stable sort keeps equal keys in index order; -0.0 and +0.0 compare equal.
    ids = np.argsort(-L.astype(np.float64), axis=1, kind="stable")[:, :k].astype(np.int32)
    sel = np.take_along_axis(L, ids, axis=1).astype(np.float64)
    z = np.exp(sel - sel[:, :1])
    w = z / z.sum(axis=1, keepdims=True)
    return ids, w


def router_projection(x_bits: np.ndarray, wr_bits: np.ndarray) -> np.ndarray:
    """R8: router logits [T][E] = x . w_r^T on the bf16 values, in float64."""
    return bf16_to_f64(x_bits) @ bf16_to_f64(wr_bits).T


# ------------------------------------------------------------- permutation --
def permute(ids: np.ndarray, E: int) -> dict:
    """Group the T*k routed slots by expert (R3).
    expert_offsets [E+1]: exclusive prefix sum of per-expert counts.
    sorted_slot [R]: flat slot f = t*k + j at each position of the grouped order
                     (stable: within an expert, f increases).
    slot_pos [R]:    inverse map, slot_pos[sorted_slot[p]] = p.
    active:          experts with at least one slot, ascending."""
    eid = np.asarray(ids, dtype=np.int64).reshape(-1)
    R = eid.size
    counts = np.bincount(eid, minlength=E)[:E]
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_slot = np.argsort(eid, kind="stable")
    slot_pos = np.empty(R, dtype=np.int64)
    slot_pos[sorted_slot] = np.arange(R)
    active = np.nonzero(counts)[0]
    return {
        "expert_offsets": offsets.astype(np.int32),
        "sorted_slot": sorted_slot.astype(np.int32),
        "slot_pos": slot_pos.astype(np.int32),
        "active": active.astype(np.int32),
        "n_active": int(active.size),
        "counts": counts.astype(np.int32),
    }


# --------------------------------------------------------------------- FFN --
def silu(g: np.ndarray) -> np.ndarray:
    return g / (1.0 + np.exp(-g))


def expert_ffn(X: np.ndarray, W13: np.ndarray, W2: np.ndarray) -> np.ndarray:
    """One expert on its rows, float64: gate/up projection, SwiGLU (R5), down."""
    I = W13.shape[0] // 2
    G = X @ W13[:I].T
    U = X @ W13[I:].T
    return (silu(G) * U) @ W2.T


def ffn_w4a16(x_bits: np.ndarray, perm: dict, k: int, get_expert) -> np.ndarray:
    """Grouped W4A16 FFN over the routed rows, in grouped (permuted) order.
    ``get_expert(e) -> (w13, s13, w2, s2)`` returns one expert's packed tensors;
    each active expert is dequantized on its own, never the whole layer.
    Returns Y float64 [R, H]: row p is the expert output for slot sorted_slot[p]."""
    X = bf16_to_f64(x_bits)
    off = perm["expert_offsets"]
    R = int(off[-1])
    Y = None
    for e in perm["active"]:
        w13, s13, w2, s2 = get_expert(int(e))
        W13 = dequant_w4(w13, s13)
        W2 = dequant_w4(w2, s2)
        if Y is None:
            Y = np.zeros((R, W2.shape[0]))
        rows = perm["sorted_slot"][off[e]:off[e + 1]]
        Y[off[e]:off[e + 1]] = expert_ffn(X[rows // k], W13, W2)
    if Y is None:
        Y = np.zeros((0, X.shape[1]))
    return Y


def combine(Y: np.ndarray, slot_pos: np.ndarray, w: np.ndarray) -> np.ndarray:
    """out[t] = sum_j w[t, j] * Y[slot_pos[t*k + j]], accumulated in increasing j (R6)."""
    T, k = w.shape
    H = Y.shape[1]
    out = np.zeros((T, H))
    pos = np.asarray(slot_pos).reshape(T, k)
    for j in range(k):
        out += w[:, j:j + 1] * Y[pos[:, j]]
    return out


# -------------------------------------------------------------------- W8A8 --
def quant_rows_int8(a: np.ndarray):
    """Dynamic per-row int8 quantization (R7), decided in float32:
    s = float32(absmax) / 127 (IEEE float32 division), q = rint(x / s) with
    round-half-even, clamped to [-127, 127]; a zero row gets s = 0, q = 0."""
    a32 = np.asarray(a, dtype=np.float32)
    amax = np.max(np.abs(a32), axis=-1) if a32.shape[-1] else np.zeros(a32.shape[:-1], np.float32)
    s = (amax.astype(np.float32) / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    r = np.rint((a32 / safe[..., None]).astype(np.float32))
    q = np.clip(r, -127, 127)
    q = np.where(s[..., None] > 0, q, 0).astype(np.int8)
    return q, s


def int_matmul_exact(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """A @ B.T on integer-valued int8 operands, exact, as int64. Done in float64:
    with |partial sums| <= K*127*127 < 2**53 every order of summation is exact."""
    Af = np.asarray(A, dtype=np.float64)
    Bf = np.asarray(B, dtype=np.float64)
    assert Af.shape[-1] * 127 * 127 < 2 ** 53
    return (Af @ Bf.T).astype(np.int64)


def ffn_w8a8(x_bits: np.ndarray, perm: dict, k: int, get_expert) -> dict:
    """Grouped W8A8 FFN (R7): per-token int8 x, int8 x int8 -> exact int32
    gate/up accumulators, float dequant + SwiGLU, per-row int8 h, exact int32
    down accumulators, y = acc2 * hs * s2. Rows in grouped order.
    ``get_expert(e) -> (w13 int8 [2I,H], s13 f32 [2I], w2 int8 [H,I], s2 f32 [H])``."""
    X = bf16_to_f64(x_bits).astype(np.float32)   # exact: bf16 values are float32 values
    xq, xs = quant_rows_int8(X)
    off = perm["expert_offsets"]
    R = int(off[-1])
    H = X.shape[1]
    out = {"xq": xq, "xs": xs}
    acc13 = h = hq = hs = acc2 = Y = None
    for e in perm["active"]:
        w13, s13, w2, s2 = get_expert(int(e))
        I = w13.shape[0] // 2
        if acc13 is None:
            acc13 = np.zeros((R, 2 * I), np.int64)
            h = np.zeros((R, I))
            hq = np.zeros((R, I), np.int8)
            hs = np.zeros(R, np.float32)
            acc2 = np.zeros((R, H), np.int64)
            Y = np.zeros((R, H))
        a, b = off[e], off[e + 1]
        tok = perm["sorted_slot"][a:b] // k
        A13 = int_matmul_exact(xq[tok], w13)
        acc13[a:b] = A13
        GU = A13.astype(np.float64) * xs[tok].astype(np.float64)[:, None] * s13.astype(np.float64)[None, :]
        he = silu(GU[:, :I]) * GU[:, I:]
        h[a:b] = he
        hq[a:b], hs[a:b] = quant_rows_int8(he.astype(np.float32))
        A2 = int_matmul_exact(hq[a:b], w2)
        acc2[a:b] = A2
        Y[a:b] = A2.astype(np.float64) * hs[a:b].astype(np.float64)[:, None] * s2.astype(np.float64)[None, :]
    out.update(acc13=acc13, h=h, hq=hq, hs=hs, acc2=acc2, y=Y)
    return out


# -------------------------------------------------------------------- W4A8 --
def group_int_dots(codes: np.ndarray, Q: np.ndarray) -> np.ndarray:
    """[rows][N][G]: exact integer dot products of int8 activation codes
    [rows][K] with int weights Q [N][K], one per 128-wide K group."""
    G = Q.shape[1] // GROUP
    out = np.zeros((codes.shape[0], Q.shape[0], G), np.int64)
    for g in range(G):
        sl = slice(g * GROUP, (g + 1) * GROUP)
        out[:, :, g] = int_matmul_exact(codes[:, sl], Q[:, sl])
    return out


def ffn_w4a8(x_bits: np.ndarray, perm: dict, k: int, get_expert) -> dict:
    """Grouped W4A8 FFN (R9). Rows in grouped order.
    ``get_expert(e) -> (w13 packed [2I,H/2], s13 fp16 bits [2I,H/128],
    w2 packed [H,I/2], s2 fp16 bits [H,I/128])`` (the W4A16 storage)."""
    X = bf16_to_f64(x_bits).astype(np.float32)
    xq, xs = quant_rows_int8(X)
    off = perm["expert_offsets"]
    R = int(off[-1])
    H = X.shape[1]
    out = {"xq": xq, "xs": xs}
    h = hq = hs = Y = None
    for e in perm["active"]:
        w13, s13, w2, s2 = get_expert(int(e))
        Q13 = unpack_int4(w13).astype(np.int64) - ZERO_POINT
        Q2 = unpack_int4(w2).astype(np.int64) - ZERO_POINT
        I = Q13.shape[0] // 2
        if h is None:
            h = np.zeros((R, I))
            hq = np.zeros((R, I), np.int8)
            hs = np.zeros(R, np.float32)
            Y = np.zeros((R, H))
        a, b = off[e], off[e + 1]
        tok = perm["sorted_slot"][a:b] // k
        A13 = group_int_dots(xq[tok], Q13)                        # [rows, 2I, G]
        GU = (A13 * fp16_to_f64(s13)[None, :, :]).sum(axis=2)
        GU *= xs[tok].astype(np.float64)[:, None]
        he = silu(GU[:, :I]) * GU[:, I:]
        h[a:b] = he
        hq[a:b], hs[a:b] = quant_rows_int8(he.astype(np.float32))
        A2 = group_int_dots(hq[a:b], Q2)                          # [rows, H, I/128]
        Y[a:b] = (A2 * fp16_to_f64(s2)[None, :, :]).sum(axis=2) * hs[a:b].astype(np.float64)[:, None]
    out.update(h=h, hq=hq, hs=hs, y=Y)
    return out


# --------------------------------------------------------------- telemetry --
def expert_loads(ids: np.ndarray, E: int) -> np.ndarray:
    """R10: routed rows per expert of one layer call (int64 [E])."""
    loads = np.zeros(E, np.int64)
    for e in np.asarray(ids).ravel():
        loads[int(e)] += 1
    return loads


def hot_rank(loads: np.ndarray, n: int) -> np.ndarray:
    """R10: the n experts with the largest load, in descending order of load,
    ties to the lower expert index (int32 [n])."""
    loads = np.asarray(loads)
    order = sorted(range(loads.shape[0]), key=lambda e: (-int(loads[e]), e))
    return np.asarray(order[:n], np.int32)


# ------------------------------------------------------------ whole layer --
def moe_layer_w4a16(x_bits, logits, k, get_expert) -> dict:
    ids, w = route_topk(logits, k)
    E = np.asarray(logits).shape[1]
    perm = permute(ids, E)
    Y = ffn_w4a16(x_bits, perm, k, get_expert)
    out = combine(Y, perm["slot_pos"], w)
    return {"ids": ids, "w": w, "perm": perm, "y": Y, "out": out}


def moe_layer_w8a8(x_bits, logits, k, get_expert) -> dict:
    ids, w = route_topk(logits, k)
    E = np.asarray(logits).shape[1]
    perm = permute(ids, E)
    r = ffn_w8a8(x_bits, perm, k, get_expert)
    out = combine(r["y"], perm["slot_pos"], w)
    r.update(ids=ids, w=w, perm=perm, out=out)
    return r


def moe_layer_w4a8(x_bits, logits, k, get_expert) -> dict:
    ids, w = route_topk(logits, k)
    E = np.asarray(logits).shape[1]
    perm = permute(ids, E)
    r = ffn_w4a8(x_bits, perm, k, get_expert)
    out = combine(r["y"], perm["slot_pos"], w)
    r.update(ids=ids, w=w, perm=perm, out=out)
    return r
