"""Fold / unfold between row-major [E, R, C] and 128x128-block-contiguous order.
Test infrastructure only.

[FP8-ZeRO1] section "参数布局变换": fold turns a row-major weight into a
sequence of 128x128 units, each stored contiguously; unfold is its inverse.
The printed form views [E, R, C] as [E, R/128, 128, C/128, 128], swaps the
two middle axes and flattens to [-1, 128, 128].  For a param whose R or C is
not a multiple of 128 the padding of section "块粒度切分" comes first (zeros
at the high end of each dimension); unfold drops it again.

These functions write the definition out block by block: block b of a param
is the padded sub-matrix [128*br : 128*br+128, 128*bc : 128*bc+128] of
expert e.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from .table import B, grid


def fold_param(w: np.ndarray) -> np.ndarray:
    """[E, R, C] -> [E*Rb*Cb, 128, 128], zero-padded, blocks in (e, br, bc) order."""
    e_n, r, c = w.shape
    _, rb, cb = grid(w.shape)
    out = np.zeros((e_n * rb * cb, B, B), dtype=w.dtype)
    k = 0
    for e in range(e_n):
        for br in range(rb):
            for bc in range(cb):
                sub = w[e, B * br:B * br + B, B * bc:B * bc + B]
                out[k, :sub.shape[0], :sub.shape[1]] = sub
                k += 1
    return out


def unfold_param(blocks: np.ndarray, shape) -> np.ndarray:
    """Inverse of fold_param: [E*Rb*Cb, 128, 128] -> [E, R, C] (padding dropped)."""
    e_n, r, c = shape
    _, rb, cb = grid(shape)
    out = np.empty((e_n, r, c), dtype=blocks.dtype)
    k = 0
    for e in range(e_n):
        for br in range(rb):
            for bc in range(cb):
                vr, vc = min(B, r - B * br), min(B, c - B * bc)
                out[e, B * br:B * br + vr, B * bc:B * bc + vc] = blocks[k, :vr, :vc]
                k += 1
    return out


def fold_shard(tab: dict, src: Dict[int, np.ndarray], dtype=np.float32) -> np.ndarray:
    """The rank's folded shard [slots, 128, 128] from row-major params.

    ``src`` maps param id -> row-major [E, R, C] array (only params the shard
    touches are needed).  Padding positions and padding slots are +0."""
    ent = tab["entries"]
    out = np.zeros((len(ent), B, B), dtype=dtype)
    for s, t in enumerate(ent):
        p = int(t["param"])
        if p < 0:
            continue
        e, br, bc, vr, vc = int(t["expert"]), int(t["brow"]), int(t["bcol"]), int(t["vrows"]), int(t["vcols"])
        out[s, :vr, :vc] = src[p][e, B * br:B * br + vr, B * bc:B * bc + vc]
    return out


def unfold_shard(tab: dict, folded: np.ndarray, dst: Dict[int, np.ndarray],
                 scales: Optional[np.ndarray] = None, dst_scales: Optional[Dict[int, np.ndarray]] = None) -> None:
    """Write the shard's valid positions back into row-major params (in place).

    ``dst`` maps param id -> row-major [E, R, C]; ``dst_scales`` maps
    param id -> [E, Rb, Cb] and receives scales[slot] at the slot's block."""
    ent = tab["entries"]
    for s, t in enumerate(ent):
        p = int(t["param"])
        if p < 0:
            continue
        e, br, bc, vr, vc = int(t["expert"]), int(t["brow"]), int(t["bcol"]), int(t["vrows"]), int(t["vcols"])
        dst[p][e, B * br:B * br + vr, B * bc:B * bc + vc] = folded[s, :vr, :vc]
        if scales is not None and dst_scales is not None:
            dst_scales[p][e, br, bc] = scales[s]


def valid_mask(tab: dict) -> np.ndarray:
    """bool [slots, 128, 128]: True where a slot position holds a real element."""
    ent = tab["entries"]
    mask = np.zeros((len(ent), B, B), dtype=bool)
    for s, t in enumerate(ent):
        if int(t["param"]) >= 0:
            mask[s, :int(t["vrows"]), :int(t["vcols"])] = True
    return mask


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 (uint16 bit patterns) -> float32: a bfloat16 is the upper half of a float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
