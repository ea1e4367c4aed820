"""Pins of the oracle's composite step: the sharded route equals the plain row-major
definition over all ranks; skip and padding invariants."""
import numpy as np
import pytest

import synth
from oracle import layout, optim, step, table
from tests import harness


def _compare_all_ranks(w):
    un = harness.run_unsharded(w)
    sh, tabs = harness.run_sharded_all_ranks(w)
    for t in range(w.steps):
        ref = un[t]
        for key in ("step", "k", "loss_scale", "found_inf", "good_steps", "skipped_total", "step_size"):
            vals = {sh[r][t]["state"][key] for r in range(w.dp)}
            assert vals == {ref["state"][key]}, (t, key, vals, ref["state"][key])
        for name, ref_name, dt in (("master", "masters", np.float32), ("m", "ms", np.float32),
                                   ("v", "vs", np.float32), ("codes", "codes", np.uint8)):
            if ref[ref_name] is None:
                continue
            got, sc = harness.unfold_all_ranks(w, tabs, {r: sh[r][t][name] for r in range(w.dp)}, dt,
                                               scales={r: sh[r][t]["scales"] for r in range(w.dp)})
            for p in range(w.n_params):
                assert got[p].tobytes() == ref[ref_name][p].tobytes(), (t, name, p)
                if name == "codes":
                    assert sc[p].tobytes() == ref["scales"][p].tobytes(), (t, "scales", p)
    return un, sh


@pytest.mark.parametrize("name", ["tiny", "tiny_clip", "tiny_lossscale", "dense_small", "moe_small", "full_small",
                                  "tiny_pow2", "ragged_small_pow2"])
def test_sharded_equals_unsharded(name):
    _compare_all_ranks(synth.get(name))


@pytest.mark.parametrize("split", ["block", "param"])
def test_sharded_equals_unsharded_ragged(split):
    _compare_all_ranks(synth.get("ragged_small").with_(split=split))


def test_clip_is_active_in_clip_workloads():
    for name in ("tiny_clip", "dense_small"):
        un = harness.run_unsharded(synth.get(name))
        assert all(0 < s["state"]["k"] < 1 for s in un), name


def test_skip_leaves_everything_unchanged():
    w = synth.get("tiny_lossscale")
    un, sh = _compare_all_ranks(w)
    skipped = [t for t in range(w.steps) if un[t]["state"]["found_inf"]]
    assert skipped == [1]  # the +inf block is injected at step 2
    t = skipped[0]
    for r in range(w.dp):
        a, b = sh[r][t - 1], sh[r][t]
        for key in ("master", "m", "v", "codes", "scales"):
            assert a[key].tobytes() == b[key].tobytes()
        assert b["state"]["step"] == a["state"]["step"]
        assert b["state"]["loss_scale"] == a["state"]["loss_scale"] / 2


def test_padding_is_masked_not_assumed_zero():
    """NaN in the grad padding and NaN-payload sentinels in master/m/v padding: no skip,
    sentinels bit-unchanged, codes 0 in padding, results equal to the clean run."""
    w = synth.get("tiny_clip")
    tab = table.build(w.shapes, w.dp, 1)
    mask = layout.valid_mask(tab)
    P = harness.masters(w)
    G = harness.grads(w, 1)
    g = layout.fold_shard(tab, G)
    p = layout.fold_shard(tab, P)
    n = tab["shard_slots"]
    z = np.zeros((n, 128, 128), np.float32)
    codes = np.zeros((n, 128, 128), np.uint8)
    sc = np.zeros(n, np.float32)
    st0 = optim.init_state(w.hp)
    clean = step.step_sharded(tab, w.hp, st0, g, p, z, z, codes, sc)
    g2, p2, m2, v2 = g.copy(), p.copy(), z.copy(), z.copy()
    g2[~mask] = np.nan
    sentinel = np.array([0x7FC0BEEF], np.uint32).view(np.float32)[0]
    for a in (p2, m2, v2):
        a[~mask] = sentinel
    dirty = step.step_sharded(tab, w.hp, st0, g2, p2, m2, v2, codes, sc)
    assert dirty[0]["found_inf"] == 0
    for i in (1, 2, 3):
        assert (dirty[i].view(np.uint32)[~mask] == 0x7FC0BEEF).all()
        assert dirty[i][mask].tobytes() == clean[i][mask].tobytes()
    assert dirty[4].tobytes() == clean[4].tobytes() and dirty[5].tobytes() == clean[5].tobytes()
    assert (dirty[4][~mask] == 0).all()


def test_padding_slots_get_unit_scale_and_zero_codes():
    w = synth.get("ragged_small")
    tab = table.build(w.shapes, w.dp, w.dp - 1)
    ent = tab["entries"]
    assert (ent["param"] < 0).any()
    P = harness.masters(w)
    g = layout.fold_shard(tab, harness.grads(w, 1))
    p = layout.fold_shard(tab, P)
    n = tab["shard_slots"]
    z = np.zeros((n, 128, 128), np.float32)
    out = step.step_sharded(tab, w.hp, optim.init_state(w.hp), g, p, z, z, np.full((n, 128, 128), 7, np.uint8),
                            np.zeros(n, np.float32))
    pad = ent["param"] < 0
    assert (out[5][pad] == 1.0).all() and (out[4][pad] == 0).all()


def test_k_override_enters_where_the_grad_is_scaled():
    """The second stage of the clip check re-runs the step with a given clip-and-unscale
    factor k.  Scaling by a power of two is exact, so the step with factor 2k on grads g
    must equal the step with factor k on grads 2g bit for bit (no overflow or subnormal
    grads here); and the factor the finalize derives, given back as k, changes nothing."""
    w = synth.get("tiny_clip")
    tab = table.build(w.shapes, w.dp, 1, table.BLOCK)
    n = tab["shard_slots"]
    P = layout.fold_shard(tab, harness.masters(w))
    g = layout.fold_shard(tab, harness.grads(w, 1))
    z = np.zeros((n, 128, 128), np.float32)
    codes, sc = np.zeros((n, 128, 128), np.uint8), np.zeros(n, np.float32)
    st0 = optim.init_state(w.hp)
    base = step.step_sharded(tab, w.hp, st0, g, P, z, z, codes, sc, extra_sumsq=3.0)
    k = base[0]["k"]
    assert 0 < k < 1
    same = step.step_sharded(tab, w.hp, st0, g, P, z, z, codes, sc, extra_sumsq=3.0, k=k)
    for a, b in zip(base[1:], same[1:]):
        assert a.tobytes() == b.tobytes()
    k2 = float(np.float32(2 * k))
    x = step.step_sharded(tab, w.hp, st0, g, P, z, z, codes, sc, extra_sumsq=3.0, k=k2)
    y = step.step_sharded(tab, w.hp, st0, (2 * g).astype(np.float32), P, z, z, codes, sc, extra_sumsq=3.0, k=k)
    assert x[0]["k"] == k2 and y[0]["k"] == k
    for a, b in zip(x[1:], y[1:]):
        assert a.tobytes() == b.tobytes()
    assert x[1].tobytes() != base[1].tobytes()  # the factor is used


def test_two_stage_clip_check_accepts_a_sum_order_flip_only():
    """The harness's stage 1 on a global sum placed where the float32 rounding of k
    flips: a GPU sum 1e-13 away (another summation order) with the k its own finalize
    gives is accepted and returned for stage 2; a k that does not follow from the GPU's
    sum, or a sum outside 1e-12, is rejected."""
    w = synth.get("tiny_clip")
    hp = w.hp
    st0 = optim.init_state(hp)
    # c = max_norm / (sqrt(G) + 1e-6) lands on the midpoint of two float32 values
    lo = np.float32(0.3)
    hi = np.nextafter(lo, np.float32(1))
    mid = (float(lo) + float(hi)) / 2
    G = (float(np.float32(hp.max_grad_norm)) / mid - 1e-6) ** 2
    ks = {}
    for d in (-1e-13, 1e-13):
        ks[d] = optim.finalize(st0, hp, G * (1 + d), 0.0)["k"]
    assert ks[-1e-13] != ks[1e-13], "the test sum must sit on a rounding boundary"
    want = optim.finalize(st0, hp, G * (1 - 1e-13), 0.0)
    got = dict(want, global_sumsq=G * (1 + 1e-13), k=ks[1e-13])
    assert harness.clip_stage1(hp, st0, got, want) == ks[1e-13]
    assert harness.clip_stage1(hp, st0, dict(want), want) is None
    with pytest.raises(AssertionError):  # k not derived from the GPU's own sum
        harness.clip_stage1(hp, st0, dict(want, global_sumsq=G * (1 - 1e-13), k=ks[1e-13]), want)
    with pytest.raises(AssertionError):  # sums too far apart
        harness.clip_stage1(hp, st0, dict(want, global_sumsq=G * (1 + 1e-11)), want)
    # stage 2 with the flipped k equals the oracle step given that k
    tab = table.build(w.shapes, w.dp, 1, table.BLOCK)
    prev = harness.initial_reference(w, tab)
    g = layout.fold_shard(tab, harness.grads(w, 1))
    R = harness.step_given_k(w, tab, prev, g, 0.0, ks[1e-13])
    assert R["state"]["k"] == ks[1e-13]
