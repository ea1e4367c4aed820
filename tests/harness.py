"""Helpers shared by the tests: drive the oracle over a whole workload.

Inputs come from ``synth`` (seeded generators); every expected value comes
from ``oracle`` alone.
"""
from __future__ import annotations

from typing import Dict, List

import numpy as np

import synth
from oracle import layout, optim, step, table


def split_id(w) -> int:
    return table.PARAM if w.split == "param" else table.BLOCK


def masters(w) -> Dict[int, np.ndarray]:
    """Row-major initial FP32 masters (bf16 weights widened exactly)."""
    out = {}
    for pid, (e_n, r, c) in enumerate(w.shapes):
        if w.master_dtype == "bf16":
            out[pid] = np.stack([layout.widen_bf16(synth.master_slab_bf16(w, pid, e)) for e in range(e_n)])
        else:
            out[pid] = np.stack([synth.master_slab(w, pid, e) for e in range(e_n)])
    return out


def grads(w, t: int) -> Dict[int, np.ndarray]:
    return {pid: np.stack([synth.grad_slab(w, pid, e, t) for e in range(s[0])])
            for pid, s in enumerate(w.shapes)}


def run_unsharded(w, steps: int = None) -> List[dict]:
    """Per step: dict(state, masters, ms, vs, codes, scales) of the plain row-major definition.
    After a skipped step codes/scales repeat the previous step's (None before any update)."""
    steps = steps or w.steps
    P = masters(w)
    M = {p: np.zeros_like(a) for p, a in P.items()}
    V = {p: np.zeros_like(a) for p, a in P.items()}
    st = optim.init_state(w.hp)
    codes = scales = None
    out = []
    for t in range(1, steps + 1):
        st, P, M, V, c, s = step.step_unsharded(w.hp, st, grads(w, t), P, M, V)
        if c is not None:
            codes, scales = c, s
        out.append(dict(state=st, masters=P, ms=M, vs=V, codes=codes, scales=scales))
    return out


def run_sharded_all_ranks(w, steps: int = None, ranks=None) -> Dict[int, List[dict]]:
    """Per rank, per step: the method's route on each rank's folded shard, with the
    other ranks' sums of squares passed in as ``extra_sumsq`` (the all-reduce)."""
    steps = steps or w.steps
    ranks = list(range(w.dp)) if ranks is None else list(ranks)
    sid = split_id(w)
    tabs = {r: table.build(w.shapes, w.dp, r, sid) for r in range(w.dp)}
    masks = {r: layout.valid_mask(tabs[r]) for r in range(w.dp)}
    P0 = masters(w)
    state = {}
    for r in ranks:
        n = tabs[r]["shard_slots"]
        state[r] = dict(st=optim.init_state(w.hp), master=layout.fold_shard(tabs[r], P0),
                        m=np.zeros((n, 128, 128), np.float32), v=np.zeros((n, 128, 128), np.float32),
                        codes=np.zeros((n, 128, 128), np.uint8), scales=np.zeros(n, np.float32))
    out = {r: [] for r in ranks}
    for t in range(1, steps + 1):
        G = grads(w, t)
        gf = {r: layout.fold_shard(tabs[r], G) for r in range(w.dp)}
        local = {r: optim.local_sumsq(gf[r][masks[r]]) for r in range(w.dp)}
        for r in ranks:
            extra = 0.0
            for q in range(w.dp):
                if q != r:
                    extra += local[q]
            s = state[r]
            st, mas, m, v, c, sc = step.step_sharded(tabs[r], w.hp, s["st"], gf[r], s["master"], s["m"], s["v"],
                                                     s["codes"], s["scales"], extra_sumsq=extra)
            state[r] = dict(st=st, master=mas, m=m, v=v, codes=c, scales=sc)
            out[r].append(dict(state=st, master=mas, m=m, v=v, codes=c, scales=sc, grad=gf[r], extra=extra))
    return out, tabs


def unfold_all_ranks(w, tabs, per_rank_arrays: Dict[int, np.ndarray], dtype, scales=None):
    """Concatenate ranks by unfolding each rank's shard into shared row-major arrays."""
    dst = {pid: np.zeros(s, dtype=dtype) for pid, s in enumerate(w.shapes)}
    dsc = {pid: np.zeros(table.grid(s), dtype=np.float32) for pid, s in enumerate(w.shapes)}
    for r, arr in per_rank_arrays.items():
        layout.unfold_shard(tabs[r], arr, dst, None if scales is None else scales[r], dsc)
    return dst, dsc


# ---------------------------------------------------------------- two-stage clip check
#
# The float64 sum of squares is the one result of the step whose value depends on a
# reduction order: the GPU and the oracle sum in different orders, agree to ~1e-16
# relative, and the clip-and-unscale factor k (rounded to float32) is then almost
# always equal.  Stage 1 checks the sums within 1e-12 and that the GPU's k is the
# oracle's finalize applied to the GPU's own sum; stage 2 re-runs the oracle's step
# with the GPU's k when the two k differ, and everything else must then be bit-exact.

def initial_reference(w, tab) -> dict:
    """The oracle's folded buffers and state before step 1 (the init fold of the masters)."""
    n = tab["shard_slots"]
    z = np.zeros((n, 128, 128), np.float32)
    return dict(state=optim.init_state(w.hp), master=layout.fold_shard(tab, masters(w)), m=z, v=z.copy(),
                codes=np.zeros((n, 128, 128), np.uint8), scales=np.zeros(n, np.float32))


def clip_stage1(hp, prev_state: dict, got: dict, want: dict, tag: str = ""):
    """Returns None when the GPU's k equals the oracle's, else the GPU's k after checking
    that it follows from the GPU's sum of squares (within 1e-12 of the oracle's)."""
    a, b = got["global_sumsq"], want["global_sumsq"]
    if not (np.isinf(a) and np.isinf(b)) and not (np.isnan(a) and np.isnan(b)):
        assert abs(a - b) <= 1e-12 * abs(b), (tag, "global_sumsq", a, b)
    if got["k"] == want["k"]:
        return None
    assert got["found_inf"] == want["found_inf"] == 0, (tag, "k differs on a skipped step")
    k = optim.finalize(prev_state, hp, a, 0.0)["k"]
    assert got["k"] == k, (tag, "GPU k is not the finalize of its own sum", got["k"], k)
    return got["k"]


def step_given_k(w, tab, prev: dict, grad, extra: float, k: float) -> dict:
    """Stage 2: the oracle's step from the reference buffers ``prev`` with factor k."""
    st, mas, m, v, c, sc = step.step_sharded(tab, w.hp, prev["state"], grad, prev["master"], prev["m"], prev["v"],
                                             prev["codes"], prev["scales"], extra_sumsq=extra, k=k)
    return dict(state=st, master=mas, m=m, v=v, codes=c, scales=sc, grad=grad, extra=extra)
