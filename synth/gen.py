"""Seeded synthetic inputs for one routed MoE FFN layer.

Every tensor is drawn from its own numpy PCG64 stream keyed by
``SeedSequence(0, spawn_key=(workload_id, unit, tag, expert))`` so any single
expert's weights can be regenerated alone (the large-expert workload holds
5.8 GB of packed weights per layer; the oracle never needs them all at once).

Formats produced (the layer's storage formats, not its arithmetic):
  * x: bf16 bit patterns (uint16) of float32 N(0,1) draws, rounded to nearest even.
  * router logits: float32 N(0,1) plus an optional per-expert bias.
  * W4A16 g128 weights: packed 4-bit codes, two per byte along K (low nibble =
    even k), every code uniform on {0..15}; a uniform random byte is exactly two
    independent uniform nibbles. fp16 scale bit patterns, one per
    (output row, 128-wide K group), value fp16(0.02*|N(0,1)|) with subnormals kept.
  * W8A8 weights: int8 uniform on [-127, 127] with one float32 scale per output
    row, 0.01*|N(0,1)|.
  * router projection weights (for the projection ahead of the top-k): bf16
    bit patterns [E][H] of N(0, 1/H) draws, so x . w_e is about N(0, 1) like
    the given logits.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

TAG_X, TAG_LOGITS, TAG_BIAS, TAG_W13, TAG_S13, TAG_W2, TAG_S2, TAG_WR = range(8)
GROUP = 128


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int          # seed key of the workload
    T: int            # tokens
    H: int            # hidden size
    I: int            # expert intermediate size
    E: int            # experts
    k: int            # experts per token
    fmt: str          # "w4a16" | "w4a8" | "w8a8"
    bias: str         # "none" | "normal" | "zipf"
    units: int        # layers (or decode steps) in one timed pass
    shared_weights: bool = False   # all units use the weights of unit 0

    @property
    def R(self) -> int:
        return self.T * self.k

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The layer workloads: a tiny correctness case, decode of two concurrent
# requests over 48 independent layers, a 512-token prefill over 48 layers, a
# 4096-token W8A8 prefill (rotated over 4 seeded layers so one layer's weights
# are never cache-warm), a large-expert decode over 16 steps of one layer, and
# the 512-token prefill again in the W4A8 format (int4 weights, int8
# activations).
WORKLOADS = {
    "tiny":         Workload("tiny", 1, 16, 256, 128, 8, 2, "w4a16", "none", 1),
    "decode_t2":    Workload("decode_t2", 2, 2, 2048, 768, 128, 8, "w4a16", "normal", 48),
    "prefill_t512": Workload("prefill_t512", 3, 512, 2048, 768, 128, 8, "w4a16", "normal", 48),
    # the same prompts, weights and logit noise without the per-expert bias:
    # the skew of prefill_t512 against uniform routing at equal T
    "prefill_t512_flat": Workload("prefill_t512_flat", 3, 512, 2048, 768, 128, 8, "w4a16",
                                  "none", 48),
    "w8a8_t4096":   Workload("w8a8_t4096", 4, 4096, 2048, 768, 128, 8, "w8a8", "none", 4),
    "w4a8_t512":    Workload("w4a8_t512", 7, 512, 2048, 768, 128, 8, "w4a8", "normal", 48),
    "decode_large": Workload("decode_large", 5, 2, 7168, 2048, 256, 8, "w4a16", "zipf", 16,
                             shared_weights=True),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def seed_seq(wl: Workload, unit: int, tag: int, expert: int = 0) -> np.random.SeedSequence:
    return np.random.SeedSequence(0, spawn_key=(wl.wid, unit, tag, expert))


def rng_for(wl: Workload, unit: int, tag: int, expert: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed_seq(wl, unit, tag, expert)))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits.
    Inputs here are finite draws, so no NaN handling is needed."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def x_bf16(wl: Workload, unit: int) -> np.ndarray:
    z = rng_for(wl, unit, TAG_X).standard_normal((wl.T, wl.H), dtype=np.float32)
    return bf16_bits_from_f32(z)


def expert_bias(wl: Workload, unit: int) -> np.ndarray:
    """Per-expert router bias (float64 [E]).
    normal: N(0, sd=0.5), one draw per layer. zipf: -1.1*ln(rank) over a seeded
    permutation of ranks 1..E, fixed for every step (selection odds ~ rank^-1.1)."""
    if wl.bias == "none":
        return np.zeros(wl.E)
    if wl.bias == "normal":
        return 0.5 * rng_for(wl, unit, TAG_BIAS).standard_normal(wl.E)
    if wl.bias == "zipf":
        ranks = rng_for(wl, 0, TAG_BIAS).permutation(wl.E) + 1
        return -1.1 * np.log(ranks.astype(np.float64))
    raise ValueError(wl.bias)


def router_logits(wl: Workload, unit: int) -> np.ndarray:
    z = rng_for(wl, unit, TAG_LOGITS).standard_normal((wl.T, wl.E))
    return (z + expert_bias(wl, unit)[None, :]).astype(np.float32)


def router_weights(wl: Workload, unit: int) -> np.ndarray:
    """bf16 bits [E][H] of the router projection, N(0, 1/H)."""
    z = rng_for(wl, _wunit(wl, unit), TAG_WR).standard_normal((wl.E, wl.H), dtype=np.float32)
    return bf16_bits_from_f32(z / np.float32(np.sqrt(wl.H)))


def _wunit(wl: Workload, unit: int) -> int:
    return 0 if wl.shared_weights else unit


def _dims(wl: Workload, which: str):
    if which == "w13":
        return 2 * wl.I, wl.H, TAG_W13, TAG_S13
    if which == "w2":
        return wl.H, wl.I, TAG_W2, TAG_S2
    raise ValueError(which)


def expert_w4(wl: Workload, unit: int, e: int, which: str):
    """Packed int4 codes uint8 [N, K/2] and fp16 scale bits uint16 [N, K/128]."""
    N, K, tw, ts = _dims(wl, which)
    u = _wunit(wl, unit)
    codes = np.frombuffer(rng_for(wl, u, tw, e).bytes(N * K // 2), dtype=np.uint8)
    z = rng_for(wl, u, ts, e).standard_normal((N, K // GROUP))
    scales = (0.02 * np.abs(z)).astype(np.float16).view(np.uint16)
    return codes.reshape(N, K // 2), scales


def expert_w8(wl: Workload, unit: int, e: int, which: str):
    """int8 weights [N, K] uniform on [-127, 127] and float32 scales [N]."""
    N, K, tw, ts = _dims(wl, which)
    u = _wunit(wl, unit)
    w = rng_for(wl, u, tw, e).integers(-127, 128, size=(N, K), dtype=np.int8)
    s = (0.01 * np.abs(rng_for(wl, u, ts, e).standard_normal(N))).astype(np.float32)
    return w, s


def layer_w4(wl: Workload, unit: int, experts=None):
    """Stacked W4A16 layer: w13 [E,2I,H/2] u8, s13 [E,2I,H/128] u16,
    w2 [E,H,I/2] u8, s2 [E,H,I/128] u16. ``experts`` limits which experts are
    drawn (others left zero) — used to build only the routed ones."""
    E = wl.E
    w13 = np.zeros((E, 2 * wl.I, wl.H // 2), np.uint8)
    s13 = np.zeros((E, 2 * wl.I, wl.H // GROUP), np.uint16)
    w2 = np.zeros((E, wl.H, wl.I // 2), np.uint8)
    s2 = np.zeros((E, wl.H, wl.I // GROUP), np.uint16)

    def fill(e):
        w13[e], s13[e] = expert_w4(wl, unit, e, "w13")
        w2[e], s2[e] = expert_w4(wl, unit, e, "w2")
    _parallel(fill, range(E) if experts is None else [int(e) for e in experts])
    return w13, s13, w2, s2


def layer_w8(wl: Workload, unit: int):
    """Stacked W8A8 layer: w13 [E,2I,H] i8, s13 [E,2I] f32, w2 [E,H,I] i8, s2 [E,H] f32."""
    E = wl.E
    w13 = np.empty((E, 2 * wl.I, wl.H), np.int8)
    s13 = np.empty((E, 2 * wl.I), np.float32)
    w2 = np.empty((E, wl.H, wl.I), np.int8)
    s2 = np.empty((E, wl.H), np.float32)

    def fill(e):
        w13[e], s13[e] = expert_w8(wl, unit, e, "w13")
        w2[e], s2[e] = expert_w8(wl, unit, e, "w2")
    _parallel(fill, range(E))
    return w13, s13, w2, s2


def _parallel(fn, items) -> None:
    """Run fn over items on a few threads (numpy's generators release the GIL
    for bulk draws); each item writes its own slice, so order does not matter."""
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(fn, items))
