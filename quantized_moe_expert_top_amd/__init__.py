"""Routed MoE FFN over group-quantized experts on MI355X (gfx950).

The layer runs as five calls into libmoe (HIP kernels behind a C ABI):
route_topk -> permute -> grouped_w4a16_ffn | grouped_w8a8_ffn -> combine.
PyTorch only provides device memory and the stream.
"""
from __future__ import annotations

from dataclasses import dataclass

from . import _lib
from ._lib import (  # noqa: F401
    MoeError, combine, expert_counts_accumulate, expert_hot_rank, grouped_w4a16_ffn, grouped_w4a8_ffn, grouped_w8a8_ffn, layer_w4a16,
    layer_w4a16_noalloc, layer_w4a16_workspace, load, permute, permute_workspace, route_topk,
    router_logits,
    w4a16_workspace, w4a8_workspace, w8a8_workspace,
)

__all__ = ["MoeError", "LayerBuffers", "moe_forward", "moe_layer", "load", "router_logits",
           "route_topk",
           "permute", "grouped_w4a16_ffn", "grouped_w4a8_ffn", "grouped_w8a8_ffn", "combine",
           "layer_w4a16", "layer_w4a16_noalloc", "expert_counts_accumulate", "expert_hot_rank"]


@dataclass
class LayerBuffers:
    """Device buffers for one layer call (allocated once, reused across calls)."""
    T: int
    H: int
    I: int
    E: int
    k: int
    fmt: str
    ids: object
    w: object
    offsets: object
    sorted_slot: object
    slot_pos: object
    active: object
    n_active: object
    perm_ws: object
    ffn_ws: object
    layer_ws: object
    y: object
    out: object

    @classmethod
    def alloc(cls, T, H, I, E, k, fmt="w4a16", device="cuda"):
        import torch
        R = T * k
        i32 = dict(dtype=torch.int32, device=device)
        pws = _lib.permute_workspace(T, E, k)
        fws = {"w4a16": _lib.w4a16_workspace, "w4a8": _lib.w4a8_workspace,
               "w8a8": _lib.w8a8_workspace}[fmt](T, H, I, E, k)
        lws = _lib.layer_w4a16_workspace(T, H, I, E, k) if fmt == "w4a16" else 0
        return cls(
            T, H, I, E, k, fmt,
            ids=torch.empty((T, k), **i32),
            w=torch.empty((T, k), dtype=torch.float32, device=device),
            offsets=torch.empty(E + 1, **i32),
            sorted_slot=torch.empty(max(R, 1), **i32),
            slot_pos=torch.empty(max(R, 1), **i32),
            active=torch.empty(max(min(E, R), 1), **i32),
            n_active=torch.empty(4, **i32),
            perm_ws=torch.empty(max(pws, 16), dtype=torch.uint8, device=device),
            ffn_ws=torch.empty(max(fws, 16), dtype=torch.uint8, device=device),
            layer_ws=torch.empty(max(lws, 16), dtype=torch.uint8, device=device),
            y=torch.empty((max(R, 1), H), dtype=torch.float32, device=device),
            out=torch.empty((T, H), dtype=torch.float32, device=device),
        )


def moe_forward(b: LayerBuffers, x, logits, weights, debug=None, stream=None):
    """One routed MoE FFN layer: x bf16 bits (int16 [T,H]), logits f32 [T,E],
    weights = (w13, s13, w2, s2) in the layout of include/moe.h. Returns b.out."""
    shape = (b.T, b.H, b.I, b.E, b.k)
    _lib.route_topk(logits, b.k, b.ids, b.w, stream)
    _lib.permute(b.ids, b.E, b.offsets, b.sorted_slot, b.slot_pos, b.active, b.n_active,
                 b.perm_ws, stream)
    w13, s13, w2, s2 = weights
    if b.fmt == "w4a16":
        _lib.grouped_w4a16_ffn(shape, x, w13, s13, w2, s2, b.offsets, b.sorted_slot, b.active,
                               b.n_active, b.y, b.ffn_ws, stream)
    elif b.fmt == "w4a8":
        _lib.grouped_w4a8_ffn(shape, x, w13, s13, w2, s2, b.offsets, b.sorted_slot, b.active,
                              b.n_active, b.y, b.ffn_ws, debug, stream)
    else:
        _lib.grouped_w8a8_ffn(shape, x, w13, s13, w2, s2, b.offsets, b.sorted_slot, b.active,
                              b.n_active, b.y, b.ffn_ws, debug, stream)
    _lib.combine(b.y, b.slot_pos, b.w, b.out, stream)
    return b.out


def moe_layer(b: LayerBuffers, x, logits, weights, stream=None):
    """The same layer through the single whole-layer entry point
    (moe_layer_w4a16; fused kernels at decode sizes). Returns b.out."""
    if b.fmt != "w4a16":
        raise ValueError("moe_layer covers the W4A16 format")
    w13, s13, w2, s2 = weights
    _lib.layer_w4a16((b.T, b.H, b.I, b.E, b.k), logits, x, w13, s13, w2, s2, b.ids, b.w,
                     b.offsets, b.sorted_slot, b.slot_pos, b.active, b.n_active, b.y, b.out,
                     b.layer_ws, stream)
    return b.out
