"""The composite shard step, in two independent formulations.  Test infrastructure only.

[FP8-ZeRO1] section "总结": fold the master at init and shard it by blocks;
each step fold the reduced grads, slice the rank's part, update, quantize
the FP32 master into FP8 codes and block scales, gather, unfold.

``step_unsharded`` is the plain definition of the result: every param kept
row-major and whole, AdamW on every element, then one scale and one set of
codes per 128x128 block of each [R, C] slice.  Sharding and folding only
change where elements sit ([FP8-ZeRO1] sections "块粒度切分" and
"参数布局变换"; [FSDP] and [DS-ZeRO] state that the sharded update is the
same computation as the unsharded one), so this is the ground truth.

``step_sharded`` follows the method's own route on one rank's folded
shard: table -> per-slot update -> per-slot requant.  Tests check the two
against each other over all ranks.
"""
from __future__ import annotations

from typing import Dict, Optional, Tuple

import numpy as np

from . import optim, quant
from .layout import valid_mask
from .table import B, grid


def step_sharded(tab: dict, hp, state: dict, grad: np.ndarray, master: np.ndarray, m: np.ndarray,
                 v: np.ndarray, codes: np.ndarray, scales: np.ndarray,
                 extra_sumsq: float = 0.0, extra_found_inf: bool = False, k: Optional[float] = None):
    """One step on a folded shard ([slots,128,128] float32 grad/master/m/v, uint8 codes,
    float32 scales[slots]).  Returns (state, master, m, v, codes, scales) as new arrays.

    ``k``, when given, replaces the clip-and-unscale factor the finalize derives from
    the sum of squares ([DS-ZeRO] section 7).  The float64 sum is the one result of the
    step that depends on a reduction order; another order may round k to a neighbouring
    float32, and the rest of the step is then checked with that k."""
    mask = valid_mask(tab)
    local = optim.local_sumsq(grad[mask]) if optim.stats_needed(hp) else None
    st = optim.finalize(state, hp, local, extra_sumsq, extra_found_inf)
    if k is not None and not st["found_inf"]:
        st["k"] = float(np.float32(k))
    master, m, v, codes, scales = (a.copy() for a in (master, m, v, codes, scales))
    if st["found_inf"]:
        return st, master, m, v, codes, scales
    p1, m1, v1 = optim.adamw(grad[mask], master[mask], m[mask], v[mask], st, hp)
    master[mask], m[mask], v[mask] = p1, m1, v1
    ent = tab["entries"]
    for s, t in enumerate(ent):
        codes[s] = 0
        if int(t["param"]) < 0:
            scales[s] = np.float32(1.0)
            continue
        vr, vc = int(t["vrows"]), int(t["vcols"])
        q, sc = quant.requant_block(master[s, :vr, :vc], getattr(hp, "scale_rule", 0))
        codes[s, :vr, :vc] = q
        scales[s] = sc
    return st, master, m, v, codes, scales


def requant_param(p: np.ndarray, rule: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Row-major [E, R, C] float32 -> (codes [E, R, C] uint8, scales [E, Rb, Cb] float32)."""
    e_n, r, c = p.shape
    _, rb, cb = grid(p.shape)
    codes = np.zeros(p.shape, dtype=np.uint8)
    scales = np.zeros((e_n, rb, cb), dtype=np.float32)
    for e in range(e_n):
        for br in range(rb):
            for bc in range(cb):
                sl = (e, slice(B * br, B * br + B), slice(B * bc, B * bc + B))
                q, s = quant.requant_block(p[sl], rule)
                codes[sl] = q
                scales[e, br, bc] = s
    return codes, scales


def step_unsharded(hp, state: dict, grads: Dict[int, np.ndarray], masters: Dict[int, np.ndarray],
                   ms: Dict[int, np.ndarray], vs: Dict[int, np.ndarray]):
    """One step over whole row-major params (dicts param id -> [E, R, C] float32).
    Returns (state, masters, ms, vs, codes, scales) with codes/scales dicts per param."""
    pids = sorted(grads)
    if optim.stats_needed(hp):
        local = sum(optim.local_sumsq(grads[p]) for p in pids) if len(pids) > 1 else optim.local_sumsq(grads[pids[0]])
    else:
        local = None
    st = optim.finalize(state, hp, local)
    if st["found_inf"]:
        return st, {p: masters[p].copy() for p in pids}, {p: ms[p].copy() for p in pids}, \
            {p: vs[p].copy() for p in pids}, None, None
    nm, nmm, nv, codes, scales = {}, {}, {}, {}, {}
    for p in pids:
        nm[p], nmm[p], nv[p] = optim.adamw(grads[p], masters[p], ms[p], vs[p], st, hp)
        codes[p], scales[p] = requant_param(nm[p], getattr(hp, "scale_rule", 0))
    return st, nm, nmm, nv, codes, scales
