"""The seeded synthetic inputs follow their stated recipe: workload shapes and
settings, independent per-slab streams, the value distributions (normal grads,
Bernoulli outliers, one lognormal factor per expert), the ragged shape rules,
the injected +inf block, and round-to-nearest BF16 weights."""
import numpy as np
import pytest

import synth


def test_workload_shapes_and_settings():
    tiny = synth.get("tiny")
    assert tiny.shapes == ((1, 256, 384), (1, 200, 300)) and tiny.dp == 2 and tiny.ranks == (0, 1)
    assert tiny.steps == 3 and tiny.hp.lr == 1e-3 and (tiny.hp.beta1, tiny.hp.beta2) == (0.9, 0.95)
    assert tiny.hp.eps == 1e-8 and tiny.hp.weight_decay == 0.1 and tiny.seed == 0
    dense = synth.get("dense")
    assert dense.shapes == ((1, 7168, 1536), (1, 1536, 24576), (1, 7168, 512), (1, 512, 32768), (1, 16384, 7168),
                            (1, 7168, 18432), (1, 18432, 7168))
    assert (dense.dp, dense.ranks[0], dense.steps, dense.hp.max_grad_norm) == (8, 3, 10, 1.0)
    assert (dense.grad_sigma, dense.grad_outlier_p, dense.grad_outlier_mult) == (1e-4, 1e-3, 100.0)
    moe = synth.get("moe")
    assert moe.shapes == ((64, 2048, 7168), (64, 2048, 7168), (64, 7168, 2048))
    assert (moe.dp, moe.ranks[0], moe.hp.max_grad_norm, moe.hp.loss_scaling) == (8, 5, 0.0, False)
    assert moe.grad_expert_lognormal and moe.grad_sigma == 1e-4
    full = synth.get("full")
    assert full.shapes == ((32, 4096, 7168),) and full.dp == 1 and full.master_dtype == "bf16"
    assert full.hp.loss_scaling and full.hp.init_scale == 2.0 ** 16 and full.hp.max_grad_norm == 1.0
    assert full.grad_premult == 2.0 ** 16 and full.steps == 5
    # the +inf block is the shard's middle slot nb // 2 (blocks in (expert, row, col) order), at step 3
    st, p, e, br, bc = full.inf_block
    rb, cb = 4096 // 128, 7168 // 128
    assert st == 3 and p == 0 and (e * rb + br) * cb + bc == (32 * rb * cb) // 2


def test_ragged_shape_rules():
    w = synth.get("ragged")
    assert len(w.shapes) == 600 and w.dp == 16 and w.ranks[0] == 7
    es = {e for e, _, _ in w.shapes}
    assert es == {1, 8}
    for e, r, c in w.shapes:
        assert 64 <= r <= 4096 and 64 <= c <= 4096
        assert r % 128 and c % 128
    # both ends of the range are reachable, and the draw is spread over it
    rs = np.array([r for _, r, _ in w.shapes] + [c for _, _, c in w.shapes])
    assert rs.min() < 200 and rs.max() > 3900 and abs(rs.mean() - 2080) < 150
    # the shape set is a fixed function of its seed
    assert synth.ragged_shapes(0, 600, 64, 4096, (1, 8)) == w.shapes
    assert synth.ragged_shapes(1, 600, 64, 4096, (1, 8)) != w.shapes


def test_slabs_are_independent_streams():
    w = synth.get("moe_small")
    a = synth.grad_slab(w, 1, 3, 2)
    assert a.dtype == np.float32 and a.shape == (256, 384)
    # the same key gives the same bits, in any order and after other draws
    synth.grad_slab(w, 0, 0, 1)
    assert synth.grad_slab(w, 1, 3, 2).tobytes() == a.tobytes()
    # other step, expert, param or kind: other draws
    for b in (synth.grad_slab(w, 1, 3, 1), synth.grad_slab(w, 1, 4, 2), synth.grad_slab(w, 0, 3, 2)):
        assert not np.array_equal(a, b)
    assert not np.array_equal(synth.master_slab(w, 1, 3), synth.master_slab(w, 1, 4))
    # a different base seed changes everything
    assert not np.array_equal(synth.grad_slab(w.with_(seed=1), 1, 3, 2), a)


def test_normal_grads_with_bernoulli_outliers():
    w = synth.get("dense")
    g = synth.grad_slab(w, 2, 0, 1).astype(np.float64)  # [7168, 512]: 3.67 M elements
    sigma = w.grad_sigma
    big = np.abs(g) > 10 * sigma  # an N(0, sigma) value beyond 10 sigma has probability ~1e-23
    # outliers are N(0, sigma) x 100: beyond 10 sigma with probability P(|N| > 0.1) = 0.920
    frac = big.mean()
    assert 0.8e-3 < frac < 1.05e-3
    rest = g[~big]
    assert abs(rest.mean()) < 3 * sigma / np.sqrt(rest.size) * 2
    assert abs(rest.std() / sigma - 1.0) < 0.01
    assert abs(np.abs(g[big]).mean() / (100 * sigma) - 0.863) < 0.05  # E|N| given |N| > 0.1 = 2 phi(0.1) / 0.920


def test_one_lognormal_factor_per_expert():
    w = synth.get("moe")
    f = np.array([synth.expert_factor(w, 2, e) for e in range(64)])
    lf = np.log(f)
    assert abs(lf.mean()) < 0.4 and abs(lf.std() - 1.0) < 0.3  # 64 draws of N(0, 1)
    for e in (0, 5):
        s1 = synth.grad_slab(w, 2, e, 1)[:1024].std()
        s2 = synth.grad_slab(w, 2, e, 2)[:1024].std()
        # the factor is the expert's, the same at every step
        assert abs(s1 / (w.grad_sigma * f[e]) - 1.0) < 0.01
        assert abs(s2 / (w.grad_sigma * f[e]) - 1.0) < 0.01
    assert synth.expert_factor(synth.get("dense"), 0, 0) == 1.0


def test_master_draw_and_bf16_rounding():
    w = synth.get("full_small")
    x = synth.master_slab(w, 0, 1)
    assert abs(x.std() / w.master_sigma - 1.0) < 0.02
    b = synth.master_slab_bf16(w, 0, 1)
    assert b.dtype == np.uint16 and b.shape == x.shape

    def widen(u):
        return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    xd = x.astype(np.float64)
    err = np.abs(widen(b) - xd)
    # round to nearest: neither bfloat16 neighbour is closer
    for step in (-1, 1):
        nb = (b.astype(np.int32) + step).astype(np.uint16)
        assert (err <= np.abs(widen(nb) - xd)).all()


def test_injected_inf_block():
    w = synth.get("full_small")  # [4, 300, 520]: +inf block (2, 4) of expert 2 at step 3
    st, p, e, br, bc = w.inf_block
    g = synth.grad_slab(w, p, e, st)
    blk = g[128 * br:128 * (br + 1), 128 * bc:128 * (bc + 1)]
    assert blk.size > 0 and np.isposinf(blk).all()
    rest = g.copy()
    rest[128 * br:128 * (br + 1), 128 * bc:128 * (bc + 1)] = 0.0
    assert np.isfinite(rest).all()
    assert np.isfinite(synth.grad_slab(w, p, e, st - 1)).all()
    assert np.isfinite(synth.grad_slab(w, p, e + 1, st)).all()
    # the grads were made at the loss scale: std = sigma x 2^16
    assert abs(synth.grad_slab(w, p, 0, 1).std() / (w.grad_sigma * w.grad_premult) - 1.0) < 0.02


@pytest.mark.parametrize("name", sorted(synth.SMALL_WORKLOADS))
def test_small_variants_keep_their_structure(name):
    w = synth.get(name)
    assert w.steps >= 2 and len(w.ranks) >= 1 and all(0 <= r < w.dp for r in w.ranks)
    assert w.total_elems() < 50_000_000  # the oracle finishes these in seconds


def test_edge_inputs_reach_their_cases():
    """The magnitude edge inputs (one kind per block) reach what each kind is for, in the
    oracle: a scale that rounds to 0, a subnormal scale, an amax near FLT_MAX, the
    power-of-two scale clamped at 2^-127, NaN and inf grads, an all-zero block."""
    import numpy as np
    from oracle import layout, optim, step as ostep, table as otable

    kinds = [k for rows in synth.EDGE_KINDS for row in rows for k in row]
    tab = otable.build(synth.EDGE_SHAPES, 1, 0, otable.BLOCK)
    assert len(kinds) == tab["shard_slots"]
    P = {p: synth.edge_master(p) for p in range(len(synth.EDGE_SHAPES))}
    G = {p: synth.edge_grad(p, 1) for p in range(len(synth.EDGE_SHAPES))}
    gf = layout.fold_shard(tab, G)
    mask = layout.valid_mask(tab)
    for rule in (0, 1):
        hp = synth.Hparams(scale_rule=rule)
        n = tab["shard_slots"]
        z = np.zeros((n, 128, 128), np.float32)
        st, master, m, v, codes, sc = ostep.step_sharded(tab, hp, optim.init_state(hp), gf,
                                                         layout.fold_shard(tab, P), z, z,
                                                         np.zeros((n, 128, 128), np.uint8), np.zeros(n, np.float32))
        for i, k in enumerate(kinds):
            real = mask[i]
            if k == "tiny":
                assert sc[i] == (0.0 if rule == 0 else 2.0 ** -127)
                assert (master[i][real] != 0).all()  # no exact zeros (0/0 would be a NaN code)
            if k == "sub_scale" and rule == 0:
                assert 0 < sc[i] < np.finfo(np.float32).tiny
            if k == "huge":
                assert np.abs(master[i][real]).max() > 3e38 and np.isfinite(master[i][real]).all()
            if k == "e8m0_clamp" and rule == 1:
                assert sc[i] == 2.0 ** -127
            if k == "nan_grad":
                assert np.isnan(gf[i][real]).any() and np.isnan(master[i][real]).any()
            if k == "inf_grad":
                assert np.isinf(gf[i][real]).any() and np.isnan(master[i][real]).any()
            if k == "zero":
                assert sc[i] == 1.0 and (codes[i] == 0).all()
