"""FP8 E4M3 (OCP "E4M3FN") encode/decode.  Test infrastructure only.

E4M3 is the FP8 training format of [FP8-Ling] section 1.1 and of the
DeepSeek-style blockwise weights of [FP8-ZeRO1] section "Blockwise 量化".
The variant is the OCP 8-bit floating point one (OFP8, "E4M3"): 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits, no infinities, a single NaN
mantissa pattern S.1111.111, largest finite 448 = S.1111.110, smallest normal
2^-6, subnormals k * 2^-9 for k = 1..7.

Encoding rule (a reading; the pages name the format only): round to nearest,
ties to even; magnitudes at or above 448 (infinities included) saturate to
448; NaN maps to the NaN pattern with the input's sign; the sign of zero and
of values that round to zero is kept.

The encoder works in float64 with frexp/rint, written from the format's
definition (quantum of the binade, then round), not from a bit trick.
"""
from __future__ import annotations

import numpy as np

MAX = 448.0
MIN_NORMAL = 2.0 ** -6
MIN_SUBNORMAL = 2.0 ** -9
NAN_CODE = 0x7F
MAX_CODE = 0x7E


def encode(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint8 E4M3 codes, elementwise."""
    x = np.asarray(x, dtype=np.float32)
    sign = ((x.view(np.uint32) >> np.uint32(31)).astype(np.uint8)) << np.uint8(7)
    with np.errstate(invalid="ignore"):  # signalling NaNs widen to quiet NaNs, flagged below
        a = np.abs(x.astype(np.float64))
    nan = np.isnan(a)
    sat = ~nan & (a >= MAX)
    fin = ~nan & ~sat
    af = np.where(fin, a, 0.0)

    # Quantum (spacing of representable values) of the binade holding |x|:
    # 2^(floor(log2|x|) - 3) for normals, 2^-9 below the smallest normal.
    mant, expo = np.frexp(af)  # af = mant * 2^expo, mant in [0.5, 1)
    quantum = np.where(af >= MIN_NORMAL, np.ldexp(1.0, expo - 4), MIN_SUBNORMAL)
    r = np.rint(af / quantum) * quantum  # exact in float64; rint is ties-to-even

    # Code of the rounded magnitude r (r <= 448 here).
    m2, e2 = np.frexp(r)  # r = m2 * 2^e2, m2 in [0.5, 1): r = (2*m2) * 2^(e2-1)
    normal = r >= MIN_NORMAL
    exp_field = np.where(normal, e2 - 1 + 7, 0)
    man_field = np.where(normal, np.rint((2.0 * m2 - 1.0) * 8.0), np.rint(r / MIN_SUBNORMAL))
    code = (exp_field.astype(np.int64) << 3) | man_field.astype(np.int64)
    code = np.where(nan, NAN_CODE, np.where(sat, MAX_CODE, code))
    return code.astype(np.uint8) | sign


def decode(codes: np.ndarray) -> np.ndarray:
    """uint8 E4M3 codes -> float64 values (NaN for the NaN pattern)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * MIN_SUBNORMAL, np.ldexp(1.0 + m / 8.0, e - 7))
    val = np.where((c & 0x7F) == NAN_CODE, np.nan, val)
    return s * val


def ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in representable steps between two codes of the same sign (+0 == -0).

    Codes of opposite sign are measured through zero.  NaN codes compare as
    distance 0 to each other and as a large distance to anything else."""
    a = np.asarray(a, dtype=np.uint8).astype(np.int64)
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)

    def signed_rank(c):
        mag = c & 0x7F
        return np.where(c & 0x80, -mag, mag)

    d = np.abs(signed_rank(a) - signed_rank(b))
    an = (a & 0x7F) == NAN_CODE
    bn = (b & 0x7F) == NAN_CODE
    return np.where(an & bn, 0, np.where(an | bn, 1 << 20, d))
