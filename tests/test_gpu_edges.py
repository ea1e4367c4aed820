"""GPU parity at the edges of the float32 range and on non-finite grads, through the
C-ABI, on both routes (fold on read, separate fold) and both scale rules, against the
oracle's sharded step.  One kind of values per 128x128 block (synth.EDGE_KINDS):
blocks whose amax / 448 is a subnormal or rounds to 0, an amax near FLT_MAX, the
power-of-two scale clamped at 2^-127, an all-zero block, and NaN / +-inf grads with
clipping and loss scaling off (no statistics are taken, so nothing skips the step
and the non-finite values reach the master, m, v and codes).

Bit-exact everywhere except the bits of a NaN: IEEE 754 fixes neither the sign nor
the payload of a NaN that an invalid operation (inf/inf, 0*inf) produces, and the
host and the GPU differ there (x86 gives a negative default NaN, gfx950 a positive
one).  So a NaN matches any NaN (master, m, v), and the NaN codes 0x7F and 0xFF
match each other; every other bit pattern must be equal."""
import numpy as np
import pytest

import synth
from oracle import layout, optim, step as ostep, table as otable

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

STEPS = 2


def _fz():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import blockwise_fp8_zero_fold_amd as fz
    return fz


def _same_f32(got, want, what):
    g, w = np.ascontiguousarray(got), np.ascontiguousarray(want)
    gn, wn = np.isnan(g), np.isnan(w)
    assert (gn == wn).all(), f"{what}: NaN positions differ ({int((gn != wn).sum())})"
    gb, wb = g.view(np.uint32), w.view(np.uint32)
    bad = (gb != wb) & ~gn
    assert not bad.any(), f"{what}: {int(bad.sum())} elements differ, first at {np.argwhere(bad)[0].tolist()}"


def _same_codes(got, want, what):
    g, w = np.asarray(got), np.asarray(want)
    gn, wn = (g & 0x7F) == 0x7F, (w & 0x7F) == 0x7F
    assert (gn == wn).all(), f"{what}: NaN codes at different positions"
    bad = (g != w) & ~gn
    assert not bad.any(), f"{what}: {int(bad.sum())} codes differ, first at {np.argwhere(bad)[0].tolist()}"


@pytest.mark.parametrize("scale_rule", [0, 1])
@pytest.mark.parametrize("fold_on_read", [True, False])
def test_magnitude_edges_and_nonfinite_grads(fold_on_read, scale_rule):
    fz = _fz()
    from blockwise_fp8_zero_fold_amd.shard import Shard
    from tests import gpu_harness as gh

    shapes = synth.EDGE_SHAPES
    hp = synth.Hparams(scale_rule=scale_rule)  # no clipping, no loss scaling
    assert not optim.stats_needed(hp)
    tab = otable.build(shapes, 1, 0, otable.BLOCK)
    n = tab["shard_slots"]
    P = {p: synth.edge_master(p) for p in range(len(shapes))}
    tag0 = f"edges fold_on_read={fold_on_read} scale_rule={scale_rule}"
    print(f"# {tag0}: {n} slots", flush=True)

    # the oracle: the method's route on the folded shard
    st = optim.init_state(hp)
    master = layout.fold_shard(tab, P)
    m = np.zeros_like(master)
    v = np.zeros_like(master)
    codes = np.zeros(master.shape, np.uint8)
    scales = np.zeros(n, np.float32)

    sh = Shard(shapes, 1, 0)
    sh.init(fz.Hparams.make(hp), [torch.from_numpy(P[p]).cuda() for p in range(len(shapes))], fz.F32)
    _same_f32(gh.folded(sh.master, n), master, f"{tag0}: init fold")
    dst_codes = [torch.full(s, 0xA5, dtype=torch.uint8, device="cuda") for s in shapes]
    dst_scales = [torch.full(otable.grid(s), float("nan"), dtype=torch.float32, device="cuda") for s in shapes]
    for t in range(1, STEPS + 1):
        G = {p: synth.edge_grad(p, t) for p in range(len(shapes))}
        gf = layout.fold_shard(tab, G)
        st, master, m, v, codes, scales = ostep.step_sharded(tab, hp, st, gf, master, m, v, codes, scales)
        sh.step(fz.Hparams.make(hp), [torch.from_numpy(G[p]).cuda() for p in range(len(shapes))], dst_codes,
                dst_scales, fused_stats=False, fold_on_read=fold_on_read)
        torch.cuda.synchronize()
        tag = f"{tag0} step {t}"
        got = sh.read_state()
        for key in ("step", "found_inf", "k", "step_size", "bc2_sqrt", "decay"):
            assert got[key] == st[key], (tag, key, got[key], st[key])
        for name, want in (("master", master), ("m", m), ("v", v)):
            _same_f32(gh.folded(getattr(sh, name), n), want, f"{tag}: {name}")
        _same_codes(gh.folded(sh.fp8, n, np.uint8), codes, f"{tag}: codes")
        _same_f32(sh.scales.cpu().numpy()[:n], scales, f"{tag}: scales")
        # the unfolded row-major codes and scales
        want_c = {p: np.zeros(s, np.uint8) for p, s in enumerate(shapes)}
        want_s = {p: np.zeros(otable.grid(s), np.float32) for p, s in enumerate(shapes)}
        layout.unfold_shard(tab, codes, want_c, scales, want_s)
        for p in range(len(shapes)):
            _same_codes(dst_codes[p].cpu().numpy(), want_c[p], f"{tag}: unfolded codes p{p}")
            _same_f32(dst_scales[p].cpu().numpy(), want_s[p], f"{tag}: unfolded scales p{p}")
    # the cases the test is for are really there
    kinds = [k for rows in synth.EDGE_KINDS for row in rows for k in row]
    ent = tab["entries"]
    sc = {kinds[i]: float(scales[i]) for i in range(len(ent)) if kinds[i] not in ("normal",)}
    assert np.isnan(master).any() and (codes & 0x7F == 0x7F).any(), "NaN must reach master and codes"
    if scale_rule == 0:
        assert sc["tiny"] == 0.0, "tiny: amax / 448 rounds to 0"
        assert 0 < sc["sub_scale"] < np.finfo(np.float32).tiny, "sub_scale: a subnormal scale"
        assert sc["huge"] > 1e35
    else:
        assert sc["e8m0_clamp"] == 2.0 ** -127 and sc["tiny"] == 2.0 ** -127, "the E8M0 clamp"
    assert sc["zero"] == 1.0
