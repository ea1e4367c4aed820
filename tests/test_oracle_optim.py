"""Pins of the oracle's statistics, step scalars, AdamW and requantization."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import e4m3, optim, quant

HP = synth.Hparams()


def _brute_adamw_f64(g_steps, p, hp, ks):
    """Scalar float64 AdamW in its textbook bias-corrected form, one element at a time,
    from the float32 values of the hyperparameters."""
    f = lambda x: float(np.float32(x))
    lr, b1, b2, eps, wd = f(hp.lr), f(hp.beta1), f(hp.beta2), f(hp.eps), f(hp.weight_decay)
    out = []
    for x0, gs in zip(p, g_steps):
        x, m, v = float(x0), 0.0, 0.0
        for t, (g, k) in enumerate(zip(gs, ks), start=1):
            g = float(g) * k
            m = b1 * m + (1 - b1) * g
            v = b2 * v + (1 - b2) * g * g
            mhat = m / (1 - b1 ** t)
            vhat = v / (1 - b2 ** t)
            x = x * (1 - lr * wd) - lr * mhat / (math.sqrt(vhat) + eps)
        out.append((x, m, v))
    return np.array(out)


def _run_oracle(g_steps, p0, hp, clip_k=None):
    st = optim.init_state(hp)
    p = p0.astype(np.float32)
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    ks = []
    for t in range(g_steps.shape[1]):
        g = g_steps[:, t].astype(np.float32)
        st = optim.finalize(st, hp, optim.local_sumsq(g) if optim.stats_needed(hp) else None)
        ks.append(st["k"])
        p, m, v = optim.adamw(g, p, m, v, st, hp)
    return p, m, v, ks


def test_adamw_matches_float64_brute_force():
    rng = np.random.default_rng(0)
    n = 4000
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal((n, 3)) * rng.choice([1e-6, 1e-3, 1.0], (n, 1))).astype(np.float32)
    p, m, v, ks = _run_oracle(g, p0, HP)
    ref = _brute_adamw_f64(g, p0, HP, [1.0, 1.0, 1.0])
    assert np.all(np.abs(p - ref[:, 0]) <= 1e-6 * np.abs(ref[:, 0]) + 1e-6 * HP.lr)
    # m can cancel (a sum of terms of both signs): bound its error by the grads' size
    gmax = np.max(np.abs(g.astype(np.float64)), axis=1)
    assert np.all(np.abs(m - ref[:, 1]) <= 1e-6 * gmax)
    assert np.all(np.abs(v - ref[:, 2]) <= 1e-6 * np.abs(ref[:, 2]))


@pytest.mark.parametrize("kw", [dict(beta1=0.0, beta2=0.0), dict(beta1=0.99, beta2=0.9999),
                                dict(lr=0.3, weight_decay=1.0), dict(eps=1e-3, weight_decay=0.0),
                                dict(lr=1e-5, eps=1e-12, beta1=0.5, beta2=0.9)])
def test_adamw_brute_force_unusual_hyperparameters(kw):
    """The same float64 brute force with betas at 0 and near 1, a large learning rate with
    full weight decay, a large eps, a tiny learning rate and eps."""
    import dataclasses
    hp = dataclasses.replace(HP, **kw)
    rng = np.random.default_rng(1)
    n = 2000
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal((n, 3)) * rng.choice([1e-6, 1e-3, 1.0], (n, 1))).astype(np.float32)
    p, m, v, ks = _run_oracle(g, p0, hp)
    ref = _brute_adamw_f64(g, p0, hp, [1.0, 1.0, 1.0])
    lr = float(np.float32(hp.lr))
    assert np.all(np.abs(p - ref[:, 0]) <= 1e-6 * np.abs(ref[:, 0]) + 1e-6 * lr), kw
    gmax = np.max(np.abs(g.astype(np.float64)), axis=1)
    assert np.all(np.abs(m - ref[:, 1]) <= 1e-6 * gmax), kw
    assert np.all(np.abs(v - ref[:, 2]) <= 1e-6 * np.abs(ref[:, 2]) + 1e-30), kw


def test_adamw_with_clipping_matches_brute_force():
    rng = np.random.default_rng(1)
    n = 3000
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal((n, 3)) * 0.1).astype(np.float32)
    hp = synth.Hparams(max_grad_norm=1.0)
    p, m, v, ks = _run_oracle(g, p0, hp)
    norms = [math.sqrt(math.fsum(float(x) ** 2 for x in g[:, t])) for t in range(3)]
    want_k = [min(1.0, 1.0 / (nn + 1e-6)) for nn in norms]
    assert all(abs(k - w) <= 1e-7 * w for k, w in zip(ks, want_k))
    ref = _brute_adamw_f64(g, p0, hp, want_k)
    assert np.all(np.abs(p - ref[:, 0]) <= 1e-6 * np.abs(ref[:, 0]) + 1e-6 * hp.lr)


def test_first_step_closed_form():
    rng = np.random.default_rng(2)
    p = (rng.standard_normal(5000) * 0.02).astype(np.float32)
    g = (rng.standard_normal(5000) * 1e-3).astype(np.float32)
    st = optim.finalize(optim.init_state(HP), HP, None)
    p1, m1, v1 = optim.adamw(g, p, np.zeros_like(p), np.zeros_like(p), st, HP)
    want = p.astype(np.float64) * (1 - 1e-3 * 0.1) - 1e-3 * g / (np.abs(g) + 1e-8)
    # a few float32 roundings of operands of size |p| and lr (the result may cancel)
    assert np.all(np.abs(p1 - want) <= 4 * np.spacing((np.abs(p) + np.float32(1e-3)).astype(np.float32)))
    # so the first step moves every element by about lr, whatever the size of its grad
    big = np.abs(g) > 1e-4
    assert np.all(np.abs(np.abs(p1 - p * np.float32(st["decay"])) - 1e-3)[big] <= 2e-7)


def test_zero_grad_is_pure_decay():
    rng = np.random.default_rng(3)
    p = (rng.standard_normal(1000) * 0.02).astype(np.float32)
    st = optim.finalize(optim.init_state(HP), HP, None)
    z = np.zeros_like(p)
    p1, m1, v1 = optim.adamw(z, p, z, z, st, HP)
    assert p1.tobytes() == (p * np.float32(st["decay"])).tobytes()
    assert not m1.any() and not v1.any()


def test_agrees_with_torch_adamw():
    rng = np.random.default_rng(4)
    n = 20000
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    gs = (rng.standard_normal((3, n)) * 1e-3).astype(np.float32)
    tp = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.AdamW([tp], lr=1e-3, betas=(0.9, 0.95), eps=1e-8, weight_decay=0.1, foreach=False)
    st = optim.init_state(HP)
    p, m, v = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
    for t in range(3):
        tp.grad = torch.from_numpy(gs[t].copy())
        opt.step()
        st = optim.finalize(st, HP, None)
        p, m, v = optim.adamw(gs[t], p, m, v, st, HP)
    ref = tp.detach().numpy()
    assert np.all(np.abs(p - ref) <= 4 * np.spacing(np.abs(ref)) + 1e-9)


def test_sumsq_matches_fsum():
    rng = np.random.default_rng(5)
    g = (rng.standard_normal(100000) * 1e-4).astype(np.float32)
    want = math.fsum(float(x) * float(x) for x in g)
    assert abs(optim.local_sumsq(g) - want) <= 1e-13 * want


def test_overflow_detection():
    hp = synth.Hparams(max_grad_norm=1.0)
    for bad in (np.inf, -np.inf, np.nan):
        g = np.ones(10, np.float32)
        g[3] = bad
        st = optim.finalize(optim.init_state(hp), hp, optim.local_sumsq(g))
        assert st["found_inf"] == 1 and st["step"] == 0 and st["skipped_total"] == 1
    # the largest float32 squared is finite in float64: no false overflow
    g = np.full(4, np.finfo(np.float32).max, np.float32)
    st = optim.finalize(optim.init_state(hp), hp, optim.local_sumsq(g))
    assert st["found_inf"] == 0 and st["step"] == 1
    # an overflow on another rank arrives through the all-reduced flag or sum
    st = optim.finalize(optim.init_state(hp), hp, 1.0, extra_found_inf=True)
    assert st["found_inf"] == 1
    st = optim.finalize(optim.init_state(hp), hp, 1.0, extra_sumsq=float("inf"))
    assert st["found_inf"] == 1


def test_loss_scale_sequence():
    """Hand-worked run: S=1024, double after 2 clean steps, halve and skip on overflow."""
    hp = synth.Hparams(loss_scaling=True, init_scale=1024.0, growth_interval=2)
    st = optim.init_state(hp)
    seq = []
    for local in (1.0, 1.0, float("inf"), 1.0, 1.0, float("nan")):
        st = optim.finalize(st, hp, local)
        seq.append((st["step"], st["loss_scale"], st["good_steps"], st["found_inf"], st["skipped_total"],
                    st["k"] if not st["found_inf"] else None))
    assert seq == [
        (1, 1024.0, 1, 0, 0, 1 / 1024),
        (2, 2048.0, 0, 0, 0, 1 / 1024),
        (2, 1024.0, 0, 1, 1, None),
        (3, 1024.0, 1, 0, 1, 1 / 1024),
        (4, 2048.0, 0, 0, 1, 1 / 1024),
        (4, 1024.0, 0, 1, 2, None),
    ]


def test_clip_and_unscale_combined():
    """Grads made at scale S: the clipped, unscaled norm is max_norm*n/(n+1e-6)."""
    hp = synth.Hparams(max_grad_norm=0.5, loss_scaling=True, init_scale=256.0)
    rng = np.random.default_rng(6)
    g_true = (rng.standard_normal(4096) * 0.05).astype(np.float32)
    g = g_true * np.float32(256.0)
    st = optim.finalize(optim.init_state(hp), hp, optim.local_sumsq(g))
    n = math.sqrt(math.fsum(float(x) ** 2 for x in g_true))
    assert n > 0.5
    clipped = np.float64(st["k"]) * g.astype(np.float64)
    got = math.sqrt(float(np.sum(clipped ** 2)))
    assert abs(got - 0.5 * n / (n + 1e-6)) <= 1e-6 * got


def test_bias_correction_scalars():
    st = optim.init_state(HP)
    for t in range(1, 6):
        st = optim.finalize(st, HP, None)
        assert st["step"] == t
        lr, b1, b2 = (float(np.float32(x)) for x in (1e-3, 0.9, 0.95))
        want = lr / (1 - b1 ** t)
        assert abs(st["step_size"] - want) <= float(np.spacing(np.float32(want)))  # one rounding
        want = math.sqrt(1 - b2 ** t)
        assert abs(st["bc2_sqrt"] - want) <= float(np.spacing(np.float32(want)))


def _quantum(y):
    a = np.abs(y)
    return np.where(a >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3), 2.0 ** -9)


def test_requant_invariants():
    rng = np.random.default_rng(7)
    for trial in range(200):
        shape = (int(rng.integers(1, 129)), int(rng.integers(1, 129)))
        x = (rng.standard_normal(shape) * 10.0 ** rng.uniform(-30, 30)).astype(np.float32)
        codes, s = quant.requant_block(x)
        amax = np.max(np.abs(x))
        assert s == np.float32(amax / np.float32(448.0))
        if s > 0 and np.isfinite(s) and s >= np.finfo(np.float32).tiny:
            assert np.max(codes & 0x7F) == 0x7E  # the largest element maps to 448
            y = (x / s).astype(np.float64)
            err = np.abs(e4m3.decode(codes) - y)
            assert np.all(err <= _quantum(y) / 2 + 1e-6 * np.abs(y))


def test_requant_special_blocks():
    c, s = quant.requant_block(np.zeros((5, 7), np.float32))
    assert s == 1.0 and not c.any()
    x = np.array([[1.0, np.nan, -2.0]], np.float32)
    c, s = quant.requant_block(x)
    assert s == np.float32(2.0) / np.float32(448.0)
    assert c[0, 1] == 0x7F and c[0, 2] == 0xFE
    c, s = quant.requant_block(np.array([[-0.0, 0.0]], np.float32))
    assert s == 1.0 and c.tolist() == [[0x80, 0x00]]


def test_quantization_health_on_synthetic_weights():
    """Underflow share and dequantization cosine ([FP8-Ling] section 1.2 health thresholds)
    on N(0, 0.02) 128x128 blocks: a sanity check of the scale rule, not a parity criterion."""
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((16, 128, 128)) * 0.02).astype(np.float32)
    zeros = 0
    cos = []
    for b in x:
        c, s = quant.requant_block(b)
        d = e4m3.decode(c) * float(s)
        zeros += int(np.sum((c & 0x7F) == 0))
        cos.append(float(np.dot(d.ravel(), b.ravel()) / (np.linalg.norm(d) * np.linalg.norm(b))))
    assert zeros / x.size < 0.005
    assert min(cos) > 0.995


def test_dequantize_closed_forms():
    codes = np.arange(256, dtype=np.uint8).reshape(1, 2, 128)
    one = np.ones((1, 1, 1), np.float32)
    d = quant.dequantize(codes, one)
    ref = e4m3.decode(codes)
    assert (np.isnan(d) == np.isnan(ref)).all() and (d[~np.isnan(d)] == ref[~np.isnan(ref)]).all()
    for k in (-40, -3, 0, 7, 30):  # a power-of-two scale only moves the exponent
        d2 = quant.dequantize(codes, np.full((1, 1, 1), 2.0 ** k, np.float32))
        fin = ~np.isnan(ref)
        assert (d2[fin] == (ref[fin] * 2.0 ** k).astype(np.float32)).all()
    # round trip: dequantize(requant(x)) is within half an E4M3 step of x, in units of the scale
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((1, 256, 384)) * 0.02).astype(np.float32)
    from oracle import step as ostep
    c, s = ostep.requant_param(x)
    y = quant.dequantize(c, s).astype(np.float64)
    sfull = np.repeat(np.repeat(s, 128, axis=1), 128, axis=2).astype(np.float64)
    q = x / sfull
    assert np.all(np.abs(y - x) <= sfull * (_quantum(q) / 2 + 1e-6 * np.abs(q)))


def test_pow2_scale_closed_forms():
    """E8M0 rule: 2^(floor(log2 amax) - 8), clamped at 2^-127; 0 -> 1; inf -> inf."""
    f = np.float32
    cases = {1.0: 2.0 ** -8, 448.0: 1.0, 500.0: 1.0, 511.9: 1.0, 512.0: 2.0, 0.75: 2.0 ** -9, 2.0 ** -100: 2.0 ** -108,
             2.0 ** -125: 2.0 ** -127, 1e-45: 2.0 ** -127, 3.0e38: 2.0 ** 119}
    for amax, want in cases.items():
        assert quant.block_scale(f(amax), quant.SCALE_POW2) == f(want), amax
    assert quant.block_scale(f(0.0), quant.SCALE_POW2) == 1.0
    assert np.isinf(quant.block_scale(f(np.inf), quant.SCALE_POW2))


def test_pow2_scale_requant_invariants():
    rng = np.random.default_rng(23)
    for _ in range(200):
        x = (rng.standard_normal((64, 96)) * 10.0 ** rng.uniform(-30, 30)).astype(np.float32)
        c, s = quant.requant_block(x, quant.SCALE_POW2)
        m, e = np.frexp(np.float64(s))
        assert m == 0.5, "a power of two"
        amax = np.max(np.abs(x).astype(np.float64))
        if s > 2.0 ** -127:
            assert 256.0 <= amax / s < 512.0
            # the largest element saturates or lands on 256..448
            assert np.max(c & 0x7F) >= 0x78
        # dividing by a power of two is exact: the codes are those of x * 2^-k
        assert (c == e4m3.encode((x.astype(np.float64) / np.float64(s)).astype(np.float32))).all()
