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

Variant scale rule (rule 1): a power-of-two scale, the E8M0 shared scale of
MXFP8 that [FP8-ZeRO1] section "Blockwise 量化" names for Blackwell, written
from the OCP microscaling definition: 2^(floor(log2 amax) - emax) with
emax = 8, the exponent of the largest E4M3 binade, kept in the E8M0 range
(clamped below at 2^-127); the block's largest magnitude then lands in
[256, 512) and the E4M3 encoder saturates it at 448.
"""
from __future__ import annotations

import numpy as np

from . import e4m3

QMAX = np.float32(448.0)


def block_amax(x: np.ndarray) -> np.float32:
    a = np.abs(np.asarray(x, dtype=np.float32)).ravel()
    return np.float32(np.fmax.reduce(a, initial=np.float32(0.0)))


SCALE_AMAX = 0
SCALE_POW2 = 1
E4M3_EMAX = 8


def block_scale(amax: np.float32, rule: int = SCALE_AMAX) -> np.float32:
    amax = np.float32(amax)
    if not amax > 0:
        return np.float32(1.0)
    if rule == SCALE_POW2:
        if np.isinf(amax):
            return amax
        _, e = np.frexp(np.float64(amax))  # amax = f * 2^e, f in [0.5, 1): floor(log2 amax) = e - 1
        return np.float32(np.ldexp(1.0, max(int(e) - 1 - E4M3_EMAX, -127)))
    with np.errstate(all="ignore"):
        return amax / QMAX


def requant_block(x: np.ndarray, rule: int = SCALE_AMAX):
    """x: the block's real elements (any shape).  Returns (codes uint8 like x, scale float32)."""
    x = np.asarray(x, dtype=np.float32)
    s = block_scale(block_amax(x), rule)
    with np.errstate(all="ignore"):
        q = x / s
    return e4m3.encode(q), np.float32(s)


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Row-major [E, R, C] codes and [E, Rb, Cb] scales -> float32 values: each code's
    exact value times its block's scale, rounded once to float32 (the product of an
    E4M3 value and a float32 is exact in float64)."""
    codes = np.asarray(codes, dtype=np.uint8)
    e_n, r, c = codes.shape
    s_full = np.repeat(np.repeat(np.asarray(scales, np.float32), 128, axis=1), 128, axis=2)[:, :r, :c]
    with np.errstate(all="ignore"):
        return (e4m3.decode(codes) * s_full.astype(np.float64)).astype(np.float32)
