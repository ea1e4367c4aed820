"""Gradient statistics, step scalars and the AdamW update.  Test infrastructure only.

Step order ([DS-ZeRO] section 3.2): global grad norm -> loss-scale update ->
unscale and clip -> optimizer step on the rank's FP32 partition.
  * Global norm ([DS-ZeRO] section 7): the L2 norm of the unscaled grads over
    the whole model; each rank contributes the sum of squares of its own
    partition and the sums are all-reduced.  Clip coefficient
    max_norm / (norm + 1e-6), applied only when it is below 1.
  * Loss scaling ([DS-ZeRO] section 6) and overflow ([DS-ZeRO] section 9 Q6):
    an inf or NaN in the grads skips the optimizer step and halves the scale;
    after a run of clean steps the scale doubles.
  * AdamW state ([FSDP] section "参数组成"; [FP8-ZeRO1] section "ZeRO-1 优化器"):
    FP32 master weights, first moment m (moving average of g) and second
    moment v (moving average of g^2).

Readings taken (none of the pages prints the optimizer formula or these
details):
  * decoupled weight decay p*(1 - lr*wd), bias correction on, eps added
    after the square root and the bias correction, in this operation order
    (every line one float32 rounding per operation):
        g   = g_raw * k
        m'  = b1*m + (1-b1)*g
        v'  = b2*v + (1-b2)*(g*g)
        den = sqrt(v') / sqrt(1 - b2^t) + eps
        p'  = p*decay - (lr / (1 - b1^t)) * (m' / den)
    k = clip_coef / S folds unscaling and clipping into one factor; S is a
    power of two, so g*(c/S) equals the two-step (g/S)*c outside subnormals.
  * Grads were made at the loss scale S in effect for this step; that S
    unscales them, and the scale update only affects the next step.
  * The sum of squares is of the grads as given (scaled by S), in float64:
    an FP32 square is exact in float64 and cannot overflow there, so the
    sum is non-finite exactly when some grad is inf or NaN.
  * A skipped step leaves t, m, v, master, codes and scales untouched.
  * Without clipping and without loss scaling no statistics are taken and
    no overflow check happens.
  * Scalars are computed in float64 from the float32 hyperparameter values
    and rounded once to float32; b1^t and b2^t are running products.
"""
from __future__ import annotations

import math

import numpy as np


def _f32(x: float) -> float:
    return float(np.float32(x))


def stats_needed(hp) -> bool:
    return hp.max_grad_norm > 0 or bool(hp.loss_scaling)


def init_state(hp) -> dict:
    return {
        "step": 0, "beta1_pow": 1.0, "beta2_pow": 1.0, "global_sumsq": 0.0,
        "loss_scale": _f32(hp.init_scale) if hp.loss_scaling else 1.0,
        "k": 1.0, "step_size": 0.0, "bc2_sqrt": 1.0, "decay": 1.0,
        "good_steps": 0, "found_inf": 0, "skipped_total": 0,
    }


def local_sumsq(g_valid: np.ndarray) -> float:
    """Sum of squares in float64 of the given FP32 grads (numpy pairwise sum)."""
    g = np.asarray(g_valid, dtype=np.float32).astype(np.float64).ravel()
    with np.errstate(over="ignore", invalid="ignore"):
        return float(np.sum(g * g))


def finalize(state: dict, hp, local, extra_sumsq: float = 0.0, extra_found_inf: bool = False) -> dict:
    """New state after this step's statistics (``local`` is None when none were taken)."""
    st = dict(state)
    scale = float(st["loss_scale"]) if hp.loss_scaling else 1.0
    if stats_needed(hp):
        glob = float(local) + float(extra_sumsq)
        found = (not math.isfinite(glob)) or bool(extra_found_inf)
    else:
        glob, found = 0.0, False
    st["global_sumsq"] = glob
    st["found_inf"] = int(found)
    if found:
        st["skipped_total"] += 1
        if hp.loss_scaling:
            st["loss_scale"] = _f32(scale * _f32(hp.backoff_factor))
            st["good_steps"] = 0
        return st
    coef = 1.0
    if hp.max_grad_norm > 0:
        norm = math.sqrt(glob) / scale
        c = _f32(hp.max_grad_norm) / (norm + 1e-6)
        if c < 1.0:
            coef = c
    st["k"] = _f32(coef / scale)
    st["step"] += 1
    st["beta1_pow"] = st["beta1_pow"] * _f32(hp.beta1)
    st["beta2_pow"] = st["beta2_pow"] * _f32(hp.beta2)
    st["step_size"] = _f32(_f32(hp.lr) / (1.0 - st["beta1_pow"]))
    st["bc2_sqrt"] = _f32(math.sqrt(1.0 - st["beta2_pow"]))
    st["decay"] = _f32(1.0 - _f32(hp.lr) * _f32(hp.weight_decay))
    if hp.loss_scaling:
        st["good_steps"] += 1
        if st["good_steps"] >= hp.growth_interval:
            st["loss_scale"] = _f32(scale * _f32(hp.growth_factor))
            st["good_steps"] = 0
    return st


def adamw(g_raw: np.ndarray, p: np.ndarray, m: np.ndarray, v: np.ndarray, st: dict, hp):
    """Elementwise AdamW in float32, one rounding per operation. Returns (p', m', v')."""
    f = np.float32
    k, decay, step_size, bc2 = f(st["k"]), f(st["decay"]), f(st["step_size"]), f(st["bc2_sqrt"])
    b1, b2, eps = f(hp.beta1), f(hp.beta2), f(hp.eps)
    omb1, omb2 = f(1.0 - float(b1)), f(1.0 - float(b2))
    g_raw, p, m, v = (np.asarray(a, dtype=np.float32) for a in (g_raw, p, m, v))
    with np.errstate(all="ignore"):
        g = g_raw * k
        m1 = b1 * m + omb1 * g
        v1 = b2 * v + omb2 * (g * g)
        den = np.sqrt(v1) / bc2 + eps
        p1 = p * decay - step_size * (m1 / den)
    return p1, m1, v1
