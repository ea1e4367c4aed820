"""Per-block requantization of the updated FP32 master.  Test infrastructure only.

[FP8-ZeRO1] section "Blockwise 量化": one scale per 128x128 block of a weight;
section "总结": after the update each rank quantizes its FP32 master into new
FP8 weights and their scales.  [FP8-Ling] section 1.2 shows the only scale
rule on the pages: scale = amax / qmax, quantized value = x / scale.

Readings taken: qmax = 448 (the largest finite E4M3 value); the scale is
stored in FP32 as the dequantization multiplier (x ~ q * scale); a block
whose amax is 0 gets scale 1 and all-zero codes; amax is a NaN-ignoring
maximum of |x| over the block's real elements (padding excluded); padding
positions get code 0x00.
"""
from __future__ import annotations

import numpy as np

from . import e4m3

QMAX = np.float32(448.0)


def block_amax(x: np.ndarray) -> np.float32:
    a = np.abs(np.asarray(x, dtype=np.float32)).ravel()
    return np.float32(np.fmax.reduce(a, initial=np.float32(0.0)))


def block_scale(amax: np.float32) -> np.float32:
    amax = np.float32(amax)
    with np.errstate(all="ignore"):
        return amax / QMAX if amax > 0 else np.float32(1.0)


def requant_block(x: np.ndarray):
    """x: the block's real elements (any shape).  Returns (codes uint8 like x, scale float32)."""
    x = np.asarray(x, dtype=np.float32)
    s = block_scale(block_amax(x))
    with np.errstate(all="ignore"):
        q = x / s
    return e4m3.encode(q), np.float32(s)
