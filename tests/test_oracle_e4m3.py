"""Pins of the oracle's E4M3 encoder against the format's definition and torch's cast."""
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import pytest

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp.txt")
CHUNK = 1 << 24


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        bits, code = line.split()[:2]
        rows.append((int(bits, 16), int(code, 16)))
    return rows


def test_ocp_closed_forms():
    rows = _golden()
    x = np.array([b for b, _ in rows], dtype=np.uint32).view(np.float32)
    want = np.array([c for _, c in rows], dtype=np.uint8)
    got = e4m3.encode(x)
    assert got.tolist() == want.tolist()


def test_decode_every_code():
    codes = np.arange(256, dtype=np.uint8)
    vals = e4m3.decode(codes)
    nan = (codes & 0x7F) == 0x7F
    assert nan.sum() == 2
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes must increase with the code"
    assert pos[0] == 0.0 and pos[1] == 2.0 ** -9 and pos[8] == 2.0 ** -6 and pos[0x7E] == 448.0
    # every finite code is a fixed point of encode(decode(.))
    fin = ~nan
    back = e4m3.encode(vals[fin].astype(np.float32))
    assert back.tolist() == codes[fin].tolist()


SUB = 1 << 18  # compared in pieces that stay in cache: ~10x faster than whole chunks


def _torch_chunk(i):
    import torch
    torch.set_num_threads(1)
    nbad, first = 0, None
    for lo in range(i * CHUNK, (i + 1) * CHUNK, SUB):
        u = np.arange(lo, lo + SUB, dtype=np.uint64).astype(np.uint32)
        x = u.view(np.float32)
        ref = torch.from_numpy(x).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        got = e4m3.encode(x)
        bad = np.nonzero(ref != got)[0]
        if len(bad) and first is None:
            first = int(u[bad[0]])
        nbad += len(bad)
    return i, nbad, first


def test_exhaustive_vs_torch_cast():
    """All 2^32 float32 bit patterns: the oracle encoder equals torch's OCP E4M3FN cast
    after clamping to +-448 (torch's cast is round-to-nearest-even but does not saturate)."""
    n_chunks = (1 << 32) // CHUNK
    workers = min(8, os.cpu_count() or 1)
    with ProcessPoolExecutor(max_workers=workers) as ex:
        results = list(ex.map(_torch_chunk, range(n_chunks)))
    bad = [(i, n, first) for i, n, first in results if n]
    assert not bad, f"mismatches (chunk, count, first bits): {bad[:5]}"


def test_half_ulp_error_bound():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(1 << 18) * rng.choice([1e-3, 1.0, 100.0], 1 << 18)).astype(np.float32)
    x = x[np.abs(x) < 448]
    q = e4m3.decode(e4m3.encode(x))
    ax = np.abs(x.astype(np.float64))
    quantum = np.where(ax >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(ax, 2.0 ** -6))) - 3), 2.0 ** -9)
    assert np.all(np.abs(q - x) <= quantum / 2)


def test_ulp_distance():
    a = np.array([0x00, 0x80, 0x01, 0x81, 0x7E, 0x7F, 0x10], dtype=np.uint8)
    b = np.array([0x80, 0x00, 0x02, 0x01, 0x7D, 0xFF, 0x10], dtype=np.uint8)
    assert e4m3.ulp_distance(a, b).tolist() == [0, 0, 1, 2, 1, 0, 0]


def test_decode_matches_torch_float8():
    """Every code's value equals torch's float8_e4m3fn -> float32 conversion."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = e4m3.decode(codes)
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == ref[~nan]).all()
    assert (np.signbit(got[~nan]) == np.signbit(ref[~nan])).all()
