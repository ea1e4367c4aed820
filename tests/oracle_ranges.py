"""The oracle's shard step over one contiguous range of slots, for runs that check
a whole full-size shard in worker processes.  Test infrastructure only: it imports
``oracle`` and ``synth`` and nothing of the library, and never touches a GPU.

Blocks are independent units of the step once the global statistics are known
([FP8-ZeRO1] section "块粒度切分"), so a shard's result is the concatenation of
the results of its slot ranges, each run with the rest of the shard's sum of
squares (plus the other ranks' sum) passed in as the extra term of the finalize.
"""
from __future__ import annotations

import hashlib
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

import synth
from oracle import layout, optim, step as ostep, table as otable


class Slabs:
    """Row-major [E, R, C] view of a param of which only some experts exist:
    ``self[e, rows, cols]`` reads (or assigns) inside expert e's [R, C] slab."""

    def __init__(self, slabs: Dict[int, np.ndarray]):
        self.slabs = slabs

    def __getitem__(self, key):
        e, rows, cols = key
        return self.slabs[e][rows, cols]

    def __setitem__(self, key, value):
        e, rows, cols = key
        self.slabs[e][rows, cols] = value


def digest(a: np.ndarray) -> str:
    return hashlib.blake2b(memoryview(np.ascontiguousarray(a)).cast("B"), digest_size=16).hexdigest()


def sub_table(name: str, rank: int, split: str, s0: int, s1: int) -> Tuple[object, dict]:
    w = synth.get(name).with_(split=split)
    tab = otable.build(w.shapes, w.dp, rank, otable.PARAM if split == "param" else otable.BLOCK)
    sub = dict(tab)
    sub["entries"] = tab["entries"][s0:s1]
    sub["shard_slots"] = s1 - s0
    return w, sub


def _touched(sub: dict) -> List[Tuple[int, int]]:
    ent = sub["entries"]
    real = ent["param"] >= 0
    return sorted({(int(p), int(e)) for p, e in zip(ent["param"][real], ent["expert"][real])})


def _fold(sub: dict, make) -> np.ndarray:
    src: Dict[int, Slabs] = {}
    for p, e in _touched(sub):
        src.setdefault(p, Slabs({})).slabs[e] = make(p, e)
    return layout.fold_shard(sub, src)


def range_sumsq(job) -> List[float]:
    """float64 sums of squares of the range's real grads, one per step."""
    name, rank, split, s0, s1, steps = job
    w, sub = sub_table(name, rank, split, s0, s1)
    mask = layout.valid_mask(sub)
    return [optim.local_sumsq(_fold(sub, lambda p, e: synth.grad_slab(w, p, e, t))[mask])
            for t in range(1, steps + 1)]


def slab_sumsq(job) -> List[float]:
    """float64 sums of squares of one expert of one param's whole grad, one per step
    (summed over all params they give every rank's grads together)."""
    name, p, e, steps = job
    w = synth.get(name)
    return [optim.local_sumsq(synth.grad_slab(w, p, e, t)) for t in range(1, steps + 1)]


STATE_KEYS = ("step", "found_inf", "skipped_total", "good_steps", "k", "loss_scale", "step_size", "bc2_sqrt",
              "decay")


def range_run(job) -> dict:
    """Init fold of the weights, then ``steps`` oracle steps on the range; returns the
    state after every step and digests of the final folded master, m, v, codes, scales.
    ``ks`` (or None): per step, a clip-and-unscale factor to use instead of the
    finalize's (the second stage of the clip check), or None for the finalize's own."""
    name, rank, split, s0, s1, steps, extras, ks = job
    w, sub = sub_table(name, rank, split, s0, s1)
    if w.master_dtype == "bf16":
        master = _fold(sub, lambda p, e: layout.widen_bf16(synth.master_slab_bf16(w, p, e)))
    else:
        master = _fold(sub, lambda p, e: synth.master_slab(w, p, e))
    n = s1 - s0
    m = np.zeros_like(master)
    v = np.zeros_like(master)
    codes = np.zeros(master.shape, np.uint8)
    scales = np.zeros(n, np.float32)
    st = optim.init_state(w.hp)
    states = []
    for t in range(1, steps + 1):
        g = _fold(sub, lambda p, e: synth.grad_slab(w, p, e, t))
        extra = 0.0 if extras is None else extras[t - 1]
        st, master, m, v, codes, scales = ostep.step_sharded(sub, w.hp, st, g, master, m, v, codes, scales,
                                                             extra_sumsq=extra, k=None if ks is None else ks[t - 1])
        del g
        states.append({k: st[k] for k in STATE_KEYS})
    return {"states": states, "master": digest(master), "m": digest(m), "v": digest(v), "codes": digest(codes),
            "scales": digest(scales)}


def ranges(nslots: int, parts: int) -> List[Tuple[int, int]]:
    per = -(-nslots // parts)
    return [(a, min(a + per, nslots)) for a in range(0, nslots, per)]


def extras_for(sums: Sequence[Sequence[float]], other: Optional[Sequence[float]] = None) -> List[List[float]]:
    """Per range and step: the sum of squares of everything outside the range (the rest of
    the shard, plus ``other`` for the other ranks).  A non-finite sum anywhere makes every
    range's extra non-finite, so every range skips that step together."""
    steps = len(sums[0])
    tot = [sum(s[t] for s in sums) + (other[t] if other is not None else 0.0) for t in range(steps)]
    out = []
    for s in sums:
        row = []
        for t in range(steps):
            row.append(tot[t] - s[t] if np.isfinite(tot[t]) else float("inf"))
        out.append(row)
    return out
