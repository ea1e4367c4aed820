"""GPU parity at the full workload sizes, in the launch configurations bench.py times
(update reading the row-major grads, or fold with fused statistics then update; then unfold):
sampled slots are checked bit for bit against the oracle, which recomputes them
one by one from the same seeded inputs; properties that hold at any size are
checked on every slot."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import synth
from oracle import layout, optim, step as ostep, table as otable
from tests import harness

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BLOCK = 128 * 128


def _fz():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import blockwise_fp8_zero_fold_amd as fz
    return fz


def _sample_slots(ent, k=32):
    n = len(ent)
    pick = set(range(min(4, n))) | set(range(max(0, n - 4), n))
    pick |= set(np.linspace(0, n - 1, k).astype(int).tolist())
    partial = np.nonzero((ent["param"] >= 0) & ((ent["vrows"] < 128) | (ent["vcols"] < 128)))[0]
    pick |= set(partial[:: max(1, len(partial) // 8)][:8].tolist())
    pad = np.nonzero(ent["param"] < 0)[0]
    pick |= set(pad[:2].tolist())
    change = np.nonzero(np.diff(ent["param"]) != 0)[0]
    for c in change[:4]:
        pick |= {int(c), int(c) + 1}
    return sorted(pick)


def _blocks_of(ent, slots, rows):
    """Folded [len(slots),128,128] float32 of the sampled slots from row-major slabs
    ``rows[(pid, e)]`` (zero padding)."""
    out = np.zeros((len(slots), 128, 128), np.float32)
    for i, s in enumerate(slots):
        t = ent[s]
        p = int(t["param"])
        if p < 0:
            continue
        e, br, bc, vr, vc = int(t["expert"]), int(t["brow"]), int(t["bcol"]), int(t["vrows"]), int(t["vcols"])
        out[i, :vr, :vc] = rows[(p, e)][128 * br:128 * br + vr, 128 * bc:128 * bc + vc]
    return out


def _slab_sumsq(ent, slab, p, e):
    """float64 sums of squares of the shard's blocks inside one row-major slab, in slot order."""
    sel = np.nonzero((ent["param"] == p) & (ent["expert"] == e))[0]
    tot = 0.0
    for s in sel:
        t = ent[s]
        br, bc, vr, vc = int(t["brow"]), int(t["bcol"]), int(t["vrows"]), int(t["vcols"])
        tot += optim.local_sumsq(slab[128 * br:128 * br + vr, 128 * bc:128 * bc + vc])
    return sel, tot


@pytest.mark.parametrize("name,steps", [("moe", 5), ("dense", 10), ("full", 5), ("ragged", 3)])
@pytest.mark.parametrize("fold_on_read", [True, False])
def test_full_size_sampled(name, steps, fold_on_read):
    fz = _fz()
    from blockwise_fp8_zero_fold_amd.shard import Shard
    from tests import gpu_harness as gh

    w = synth.get(name)
    rank = w.ranks[0]
    split = fz.SPLIT_PARAM if w.split == "param" else fz.SPLIT_BLOCK
    tab = otable.build(w.shapes, w.dp, rank, otable.PARAM if w.split == "param" else otable.BLOCK)
    ent = tab["entries"]
    sh = Shard(w.shapes, w.dp, rank, split)
    assert sh.table.entries().tobytes() == ent.tobytes()
    held = gh.held_experts(ent)
    slots = _sample_slots(ent)
    sub = dict(tab)
    sub["entries"] = ent[slots]
    sub["shard_slots"] = len(slots)
    sub_mask = layout.valid_mask(sub)
    stats = optim.stats_needed(w.hp)
    need = {(p, e) for p, es in held.items() for e in es}
    bf16 = w.master_dtype == "bf16"
    print(f"[{name}] rank {rank}: {len(ent)} slots, sample {len(slots)}", flush=True)

    def upload(make, dtype):
        out = [torch.zeros(s, dtype=dtype, device="cuda") if p in held else None for p, s in enumerate(w.shapes)]
        kept = {}
        sums = {}
        with ThreadPoolExecutor(16) as ex:
            for (p, e), slab in zip(sorted(need), ex.map(lambda pe: make(*pe), sorted(need))):
                src = torch.from_numpy(slab.view(np.int16)).view(torch.bfloat16) if dtype == torch.bfloat16 \
                    else torch.from_numpy(slab)
                out[p][e].copy_(src)
                kept[(p, e)] = layout.widen_bf16(slab) if dtype == torch.bfloat16 else slab
        return out, kept

    weights, P = upload((lambda p, e: synth.master_slab_bf16(w, p, e)) if bf16 else
                        (lambda p, e: synth.master_slab(w, p, e)), torch.bfloat16 if bf16 else torch.float32)
    sh.init(fz.Hparams.make(w.hp), weights, fz.BF16 if bf16 else fz.F32)
    del weights
    master = _blocks_of(ent, slots, P)
    del P
    n = len(slots)
    m = np.zeros((n, 128, 128), np.float32)
    v = np.zeros((n, 128, 128), np.float32)
    codes = np.zeros((n, 128, 128), np.uint8)
    sc = np.zeros(n, np.float32)
    st = optim.init_state(w.hp)
    dst_codes, dst_scales = gh.code_tensors(w, held)
    idx = torch.tensor(slots, device="cuda")

    for t in range(1, steps + 1):
        grads, G = upload(lambda p, e: synth.grad_slab(w, p, e, t), torch.float32)
        g_sub = _blocks_of(ent, slots, G)
        extra = 0.0
        if stats:
            local_full = 0.0
            for (p, e) in sorted(need):
                local_full += _slab_sumsq(ent, G[(p, e)], p, e)[1]
            local_sub = optim.local_sumsq(g_sub[sub_mask])
            other = 0.0
            if w.dp > 1:  # the other ranks' grads: all params' sums minus this shard's
                tot = 0.0
                for p, (E, R, C) in enumerate(w.shapes):
                    for e in range(E):
                        slab = G[(p, e)] if (p, e) in G else synth.grad_slab(w, p, e, t)
                        tot += optim.local_sumsq(slab)
                other = tot - local_full
            extra = (local_full - local_sub) + other
            hp = fz.Hparams.make(w.hp, extra_sumsq=other)
        else:
            hp = fz.Hparams.make(w.hp)
        del G
        sh.step(hp, grads, dst_codes, dst_scales, fused_stats=True, fold_on_read=fold_on_read)
        del grads
        torch.cuda.synchronize()
        gst = sh.read_state()
        tag = f"{name} step {t}"
        prev = (st, master, m, v, codes, sc)
        st, master, m, v, codes, sc = ostep.step_sharded(sub, w.hp, st, g_sub, master, m, v, codes, sc,
                                                         extra_sumsq=extra)
        if stats:
            # two-stage clip check: sums within 1e-12; a k that differs by the sum order is
            # checked to follow from the GPU's sum, and the oracle's step re-run with it
            k_gpu = harness.clip_stage1(w.hp, prev[0], gst, st, tag)
            if k_gpu is not None:
                st, master, m, v, codes, sc = ostep.step_sharded(sub, w.hp, *prev[:1], g_sub, *prev[1:],
                                                                 extra_sumsq=extra, k=k_gpu)
        for key in ("step", "found_inf", "k", "loss_scale", "step_size", "bc2_sqrt", "decay"):
            assert gst[key] == st[key], (tag, key, gst[key], st[key])

        def rows(x, dt=torch.float32):
            return x.view(-1, BLOCK)[idx].cpu().numpy().reshape(n, 128, 128)

        assert gh.bits_equal(rows(sh.master), master), f"{tag}: master"
        assert gh.bits_equal(rows(sh.m), m), f"{tag}: m"
        assert gh.bits_equal(rows(sh.v), v), f"{tag}: v"
        assert gh.bits_equal(rows(sh.fp8), codes), f"{tag}: codes"
        assert gh.bits_equal(sh.scales[idx].cpu().numpy(), sc), f"{tag}: scales"
        # the unfolded row-major codes and scales of the sampled blocks
        for i, s in enumerate(slots):
            e_ = ent[s]
            p = int(e_["param"])
            if p < 0:
                continue
            e, br, bc, vr, vc = (int(e_["expert"]), int(e_["brow"]), int(e_["bcol"]), int(e_["vrows"]),
                                 int(e_["vcols"]))
            got = dst_codes[p][e, 128 * br:128 * br + vr, 128 * bc:128 * bc + vc].cpu().numpy()
            assert (got == codes[i, :vr, :vc]).all(), f"{tag}: unfolded codes slot {s}"
            assert float(dst_scales[p][e, br, bc]) == float(sc[i]) or st["step"] == 0
        # properties on every slot: scales positive and finite; every real block whose scale is a
        # float32 normal has a code of magnitude 448 (its amax); padding codes are 0
        if st["step"] > 0:
            scales = sh.scales[: len(ent)]
            real = torch.from_numpy(ent["param"] >= 0).cuda()
            assert bool((scales > 0).all()) and bool(torch.isfinite(scales).all())
            mags = (sh.fp8.view(-1, BLOCK)[: len(ent)] & 0x7F).amax(dim=1)
            normal = real & (scales >= torch.finfo(torch.float32).tiny)
            assert bool((mags[normal] == 0x7E).all()), f"{tag}: a block without its amax code"
            if (~real).any():
                assert int(sh.fp8.view(-1, BLOCK)[: len(ent)][~real].sum()) == 0
        print(f"[{name}] step {t} ok (k={gst['k']:.6g}, skipped={gst['skipped_total']})", flush=True)
