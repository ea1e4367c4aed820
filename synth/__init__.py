"""Seeded synthetic inputs for the blockwise-FP8 ZeRO-1 shard step.

This module is shared by the oracle's tests and by the GPU tests and bench.
It holds workload descriptions (shapes, data-parallel size, ranks, step
counts, hyperparameter values, value distributions) and the generators that
draw their inputs.  It holds none of the method's arithmetic: no layout
transform, no shard table, no optimizer and no quantization.

Every slab is drawn from its own numpy PCG64 stream keyed by
``(seed, kind, param, expert, draw)``, so any expert of any param at any step
can be regenerated on its own, in any order, on any machine.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

KIND_MASTER = 0
KIND_GRAD = 1
KIND_FACTOR = 2
KIND_SHAPES = 3


@dataclass(frozen=True)
class Hparams:
    """AdamW / clipping / loss-scale settings, all as float32 values."""

    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1
    max_grad_norm: float = 0.0  # <= 0 turns clipping off
    loss_scaling: bool = False
    init_scale: float = 65536.0
    growth_factor: float = 2.0
    backoff_factor: float = 0.5
    growth_interval: int = 1000
    scale_rule: int = 0  # 0: amax / 448; 1: power of two (E8M0)


@dataclass(frozen=True)
class Workload:
    name: str
    shapes: Tuple[Tuple[int, int, int], ...]
    dp: int
    ranks: Tuple[int, ...]  # ranks exercised; ranks[0] is the one timed
    steps: int
    hp: Hparams
    seed: int = 0
    split: str = "block"  # "block" or "param"
    master_sigma: float = 0.02
    master_dtype: str = "f32"  # "f32" or "bf16" (bf16 weights folded at init)
    grad_sigma: float = 1e-3
    grad_outlier_p: float = 0.0  # Bernoulli probability of an outlier
    grad_outlier_mult: float = 1.0  # outliers are multiplied by this
    grad_expert_lognormal: bool = False  # one exp(N(0,1)) factor per expert
    grad_premult: float = 1.0  # e.g. the loss scale the grads were made with
    # (step, param, expert, block_row, block_col) whose whole block is +inf
    inf_block: Optional[Tuple[int, int, int, int, int]] = None

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def n_params(self) -> int:
        return len(self.shapes)

    def total_elems(self) -> int:
        return int(sum(e * r * c for e, r, c in self.shapes))


def _rng(seed: int, kind: int, pid: int, e: int, draw: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, kind, pid, e, draw]))


def master_slab(w: Workload, pid: int, e: int) -> np.ndarray:
    """Initial FP32 master of expert ``e`` of param ``pid``: N(0, master_sigma), shape [R, C]."""
    _, r, c = w.shapes[pid]
    x = _rng(w.seed, KIND_MASTER, pid, e, 0).standard_normal((r, c), dtype=np.float32)
    x *= np.float32(w.master_sigma)
    return x


def master_slab_bf16(w: Workload, pid: int, e: int) -> np.ndarray:
    """The same draw as ``master_slab`` rounded to bfloat16 (torch's RNE cast); uint16 bits."""
    import torch

    x = torch.from_numpy(master_slab(w, pid, e)).to(torch.bfloat16)
    return x.view(torch.int16).numpy().view(np.uint16).copy()


def expert_factor(w: Workload, pid: int, e: int) -> float:
    """Per-expert grad magnitude factor exp(N(0,1)) (lognormal(0,1)), fixed over steps."""
    if not w.grad_expert_lognormal:
        return 1.0
    z = _rng(w.seed, KIND_FACTOR, pid, e, 0).standard_normal()
    return float(np.float32(np.exp(z)))


def grad_slab(w: Workload, pid: int, e: int, step: int) -> np.ndarray:
    """Reduced FP32 grad of expert ``e`` of param ``pid`` at step ``step`` (1-based), shape [R, C]."""
    _, r, c = w.shapes[pid]
    rng = _rng(w.seed, KIND_GRAD, pid, e, step)
    g = rng.standard_normal((r, c), dtype=np.float32)
    scale = np.float32(w.grad_sigma * expert_factor(w, pid, e) * w.grad_premult)
    g *= scale
    if w.grad_outlier_p > 0.0:
        mask = rng.random((r, c)) < w.grad_outlier_p
        g[mask] *= np.float32(w.grad_outlier_mult)
    if w.inf_block is not None:
        st, ip, ie, br, bc = w.inf_block
        if st == step and ip == pid and ie == e:
            g[128 * br:128 * (br + 1), 128 * bc:128 * (bc + 1)] = np.inf
    return g


def ragged_shapes(seed: int, n: int, lo: int, hi: int, experts: Tuple[int, ...]) -> Tuple[Tuple[int, int, int], ...]:
    """``n`` shapes with R, C uniform integers in [lo, hi], redrawn while a multiple of 128,
    and E drawn uniformly from ``experts``."""
    rng = _rng(seed, KIND_SHAPES, n, lo, hi)
    out = []
    for _ in range(n):
        dims = []
        for _d in range(2):
            while True:
                v = int(rng.integers(lo, hi + 1))
                if v % 128 != 0:
                    break
            dims.append(v)
        e = int(experts[int(rng.integers(0, len(experts)))])
        out.append((e, dims[0], dims[1]))
    return tuple(out)


TINY_HP = Hparams()

WORKLOADS = {
    # Two FP32 masters, one of them ragged; DP=2, both ranks; 3 steps.
    "tiny": Workload(
        name="tiny", shapes=((1, 256, 384), (1, 200, 300)), dp=2, ranks=(0, 1), steps=3,
        hp=TINY_HP, grad_sigma=1e-3),
    # DeepSeek-style dense projections; DP=8 rank 3; 0.1% outliers x100; clip 1.0.
    "dense": Workload(
        name="dense",
        shapes=((1, 7168, 1536), (1, 1536, 24576), (1, 7168, 512), (1, 512, 32768),
                (1, 16384, 7168), (1, 7168, 18432), (1, 18432, 7168)),
        dp=8, ranks=(3,), steps=10, hp=dataclasses.replace(TINY_HP, max_grad_norm=1.0),
        grad_sigma=1e-4, grad_outlier_p=1e-3, grad_outlier_mult=100.0),
    # MoE expert tensors; DP=8 rank 5; per-expert lognormal grad scale; no clip.
    "moe": Workload(
        name="moe", shapes=((64, 2048, 7168), (64, 2048, 7168), (64, 7168, 2048)),
        dp=8, ranks=(5,), steps=5, hp=TINY_HP, grad_sigma=1e-4, grad_expert_lognormal=True),
    # 600 ragged params, DP=16 rank 7.
    "ragged": Workload(
        name="ragged", shapes=ragged_shapes(0, 600, 64, 4096, (1, 8)), dp=16, ranks=(7,),
        steps=3, hp=TINY_HP, grad_sigma=1e-3),
    # One [32,4096,7168] expert tensor from BF16 weights, DP=1: clip 1.0 + loss scaling,
    # grads made at scale 2^16, one +inf block at step 3 (slot nb//2 = expert 16, block (0,0)).
    "full": Workload(
        name="full", shapes=((32, 4096, 7168),), dp=1, ranks=(0,), steps=5,
        hp=dataclasses.replace(TINY_HP, max_grad_norm=1.0, loss_scaling=True, init_scale=65536.0),
        master_dtype="bf16", grad_sigma=1e-4, grad_premult=65536.0, inf_block=(3, 0, 16, 0, 0)),
}

# Reduced variants that the oracle finishes in seconds; they keep each config's
# structure (ragged edges, several ranks, clipping, loss scaling, skip).
SMALL_WORKLOADS = {
    "tiny_clip": WORKLOADS["tiny"].with_(
        name="tiny_clip", hp=dataclasses.replace(TINY_HP, max_grad_norm=0.05)),
    "tiny_lossscale": WORKLOADS["tiny"].with_(
        name="tiny_lossscale", steps=5, grad_premult=1024.0,
        hp=dataclasses.replace(TINY_HP, max_grad_norm=1.0, loss_scaling=True, init_scale=1024.0,
                               growth_interval=2),
        inf_block=(2, 1, 0, 1, 2)),
    "dense_small": Workload(
        name="dense_small", shapes=((1, 384, 256), (1, 128, 640), (1, 640, 128), (1, 256, 512)),
        dp=8, ranks=tuple(range(8)), steps=4, hp=dataclasses.replace(TINY_HP, max_grad_norm=0.1),
        grad_sigma=1e-4, grad_outlier_p=1e-3, grad_outlier_mult=100.0),
    "moe_small": Workload(
        name="moe_small", shapes=((8, 256, 384), (8, 256, 384), (8, 384, 256)),
        dp=8, ranks=tuple(range(8)), steps=3, hp=TINY_HP, grad_sigma=1e-4,
        grad_expert_lognormal=True),
    "ragged_small": Workload(
        name="ragged_small", shapes=ragged_shapes(1, 40, 64, 700, (1, 3)), dp=16,
        ranks=tuple(range(16)), steps=2, hp=TINY_HP, grad_sigma=1e-3),
    "tiny_pow2": WORKLOADS["tiny"].with_(
        name="tiny_pow2", hp=dataclasses.replace(TINY_HP, max_grad_norm=0.05, scale_rule=1)),
    "ragged_small_pow2": Workload(
        name="ragged_small_pow2", shapes=ragged_shapes(1, 40, 64, 700, (1, 3)), dp=16,
        ranks=(0, 7, 15), steps=2, hp=dataclasses.replace(TINY_HP, scale_rule=1), grad_sigma=1e-3),
    # long ragged rows (40,000 columns: one unfold work item per row of a block row)
    # next to short ones
    "wide_rows_small": Workload(
        name="wide_rows_small", shapes=((1, 150, 40000), (1, 300, 520)), dp=2, ranks=(0, 1), steps=2,
        hp=TINY_HP, grad_sigma=1e-3),
    # columns in whole 128-column blocks (every row-major block row segment starts
    # on a 128-byte line of an aligned array), ragged row counts; the full_small
    # recipe otherwise, on two ranks
    "lines_small": Workload(
        name="lines_small", shapes=((4, 300, 512), (1, 200, 256)), dp=2, ranks=(0, 1), steps=5,
        hp=dataclasses.replace(TINY_HP, max_grad_norm=1.0, loss_scaling=True, init_scale=65536.0),
        master_dtype="bf16", grad_sigma=1e-4, grad_premult=65536.0, inf_block=(3, 0, 1, 2, 3)),
    "full_small": Workload(
        name="full_small", shapes=((4, 300, 520),), dp=1, ranks=(0,), steps=5,
        hp=dataclasses.replace(TINY_HP, max_grad_norm=1.0, loss_scaling=True, init_scale=65536.0),
        master_dtype="bf16", grad_sigma=1e-4, grad_premult=65536.0, inf_block=(3, 0, 2, 2, 4)),
}


# Magnitude edge cases: one kind of master and grad values per 128x128 block, so
# that a small set reaches the ends of the float32 range and the special values.
# Block kinds (row-major over each param's block grid):
#   normal      master N(0, 0.02), grad N(0, 1e-3)
#   tiny        master +-k * 2^-149 (k in 1..100, no zeros), grad 0: the block's
#               amax / 448 is below half the smallest subnormal
#   sub_scale   master N(0, 1e-37), grad 0: amax / 448 is a subnormal
#   huge        master +-[1e38, 3.3e38], grad N(0, 1e-3): amax near FLT_MAX
#   nan_grad    master N(0, 0.02), grad N(0, 1e-3) with 1 % NaN
#   inf_grad    master N(0, 0.02), grad N(0, 1e-3) with 1 % +-inf
#   e8m0_clamp  master +-[2^-131, 1.5 * 2^-125], grad 0: the power-of-two scale
#               2^(floor(log2 amax) - 8) is below 2^-127 and clamps there
#   zero        master 0, grad 0
EDGE_SHAPES = ((1, 256, 512), (1, 200, 300))
EDGE_KINDS = (
    (("normal", "tiny", "sub_scale", "huge"), ("nan_grad", "inf_grad", "e8m0_clamp", "zero")),
    (("normal", "huge", "tiny"), ("nan_grad", "sub_scale", "e8m0_clamp")),
)


def edge_master(pid: int, seed: int = 0) -> np.ndarray:
    """Row-major [E, R, C] FP32 master of edge param ``pid`` (one kind per block)."""
    e_n, r, c = EDGE_SHAPES[pid]
    out = np.zeros((e_n, r, c), np.float32)
    for br, row in enumerate(EDGE_KINDS[pid]):
        for bc, kind in enumerate(row):
            sl = (0, slice(128 * br, min(r, 128 * br + 128)), slice(128 * bc, min(c, 128 * bc + 128)))
            shape = out[sl].shape
            rng = _rng(seed, KIND_MASTER, 1000 + pid, br, bc)
            sign = np.where(rng.random(shape) < 0.5, -1.0, 1.0).astype(np.float32)
            if kind in ("normal", "nan_grad", "inf_grad"):
                out[sl] = rng.standard_normal(shape, dtype=np.float32) * np.float32(0.02)
            elif kind == "tiny":
                k = rng.integers(1, 101, size=shape).astype(np.uint32)
                out[sl] = k.view(np.float32) * sign  # k * 2^-149: the subnormal with integer significand k
            elif kind == "sub_scale":
                out[sl] = (rng.standard_normal(shape) * 1e-37).astype(np.float32)
            elif kind == "huge":
                out[sl] = (rng.uniform(1e38, 3.3e38, size=shape) * sign).astype(np.float32)
            elif kind == "e8m0_clamp":
                out[sl] = (rng.uniform(2.0 ** -131, 1.5 * 2.0 ** -125, size=shape) * sign).astype(np.float32)
    return out


def edge_grad(pid: int, step: int, seed: int = 0) -> np.ndarray:
    """Row-major [E, R, C] FP32 grad of edge param ``pid`` at step ``step``."""
    e_n, r, c = EDGE_SHAPES[pid]
    out = np.zeros((e_n, r, c), np.float32)
    for br, row in enumerate(EDGE_KINDS[pid]):
        for bc, kind in enumerate(row):
            sl = (0, slice(128 * br, min(r, 128 * br + 128)), slice(128 * bc, min(c, 128 * bc + 128)))
            shape = out[sl].shape
            rng = _rng(seed, KIND_GRAD, 1000 + pid, 1000 * br + bc, step)
            if kind in ("normal", "huge", "nan_grad", "inf_grad"):
                g = rng.standard_normal(shape, dtype=np.float32) * np.float32(1e-3)
                hit = rng.random(shape) < 0.01
                if kind == "nan_grad":
                    g[hit] = np.nan
                elif kind == "inf_grad":
                    g[hit] = np.where(rng.random(int(hit.sum())) < 0.5, -np.inf, np.inf).astype(np.float32)
                out[sl] = g
    return out


def get(name: str) -> Workload:
    if name in WORKLOADS:
        return WORKLOADS[name]
    return SMALL_WORKLOADS[name]
