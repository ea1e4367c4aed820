"""GPU parity: the HIP path through the C-ABI against the oracle, element by element,
on seeded inputs that span several blocks, ragged tails, padding slots, clipping,
loss scaling and a skipped step."""
import os

import numpy as np
import pytest

import synth
from oracle import e4m3 as oe4m3
from oracle import layout, optim, table as otable
from tests import harness

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

fz = None


def setup_module(module):
    global fz
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import blockwise_fp8_zero_fold_amd as _fz  # raises if the library is not built
    fz = _fz
    from tests import gpu_harness  # noqa: F401


def _gh():
    from tests import gpu_harness
    return gpu_harness


# ---------------------------------------------------------------- encoder

def test_encoder_exhaustive_vs_torch_cast():
    """All 2^32 float32 patterns: the device encoder equals torch's E4M3FN cast after
    clamping to +-448 (NaN codes checked against the sign rule)."""
    chunk = 1 << 28
    out = torch.empty(chunk, dtype=torch.uint8, device="cuda")
    for i in range(16):
        lo = -(1 << 31) + i * chunk
        u = torch.arange(lo, lo + chunk, dtype=torch.int32, device="cuda")
        x = u.view(torch.float32)
        fz.fp8z1_encode_e4m3(x, out)
        ref = x.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
        nan = torch.isnan(x)
        bad = (out != ref) & ~nan
        assert int(bad.sum()) == 0, f"chunk {i}: {int(bad.sum())} mismatches"
        want_nan = torch.where(u < 0, 0xFF, 0x7F).to(torch.uint8)
        assert bool(((out == want_nan) | ~nan).all())
    torch.cuda.synchronize()


def test_encoder_matches_oracle_sample():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    # every exponent x every pattern of the top 5 mantissa bits x a few low-bit patterns x both signs
    e = np.arange(256, dtype=np.uint32)[:, None, None]
    m = (np.arange(32, dtype=np.uint32) << 18)[None, :, None]
    low = np.array([0, 1, 0x1FFFF, 0x20000, 0x3FFFF, 0x12345], dtype=np.uint32)[None, None, :]
    grid = ((e << 23) | m | low).ravel()
    bits = np.concatenate([bits, grid, grid | np.uint32(0x80000000)])
    x = bits.view(np.float32)
    xd = torch.from_numpy(x.copy()).cuda()
    out = torch.empty(len(x), dtype=torch.uint8, device="cuda")
    fz.fp8z1_encode_e4m3(xd, out)
    got = out.cpu().numpy()
    want = oe4m3.encode(x)
    assert (got == want).all(), np.nonzero(got != want)[0][:5]


# ---------------------------------------------------------------- fold / unfold

SMALL = ["tiny", "dense_small", "moe_small", "ragged_small", "full_small"]


@pytest.mark.parametrize("name", SMALL)
@pytest.mark.parametrize("split", [0, 1])
def test_fold_unfold_bit_exact(name, split):
    gh = _gh()
    w = synth.get(name)
    rng = np.random.default_rng(9)
    # random bit patterns: NaN payloads, -0, subnormals must all move unchanged
    src = {p: rng.integers(0, 2 ** 32, size=s, dtype=np.uint64).astype(np.uint32).view(np.float32)
           for p, s in enumerate(w.shapes)}
    src16 = {p: rng.integers(0, 2 ** 16, size=s, dtype=np.uint16) for p, s in enumerate(w.shapes)}
    for r in list(range(w.dp))[:4] + [otable.ALL_RANKS]:
        tab = otable.build(w.shapes, w.dp, r, split)
        t = fz.fp8z1_build_table(w.shapes, w.dp, r, split)
        n = t.shard_slots
        held = gh.held_experts(tab["entries"])
        d32 = [torch.from_numpy(src[p]).cuda() if p in held else None for p in range(w.n_params)]
        d16 = [torch.from_numpy(src16[p].view(np.int16)).cuda().view(torch.bfloat16) if p in held else None
               for p in range(w.n_params)]
        dst = torch.full((n * 16384,), float("nan"), dtype=torch.float32, device="cuda")
        fz.fp8z1_fold(t, d32, fz.F32, dst)
        want = layout.fold_shard(tab, src)
        assert gh.bits_equal(gh.folded(dst, n), want), (r, gh.first_diff(gh.folded(dst, n), want))
        # unfold into sentinel-filled arrays: held positions get the source bits back, the rest is untouched
        sentinel = np.uint32(0x7FC0DEAD)
        outs = [torch.full(s, 0, dtype=torch.int32, device="cuda").fill_(int(sentinel)).view(torch.float32)
                if p in held else None for p, s in enumerate(w.shapes)]
        fz.fp8z1_unfold(t, dst, fz.F32, None, outs)
        ones = layout.valid_mask(tab)
        for p in held:
            mask = np.zeros(w.shapes[p], bool)
            layout.unfold_shard(tab, ones, {p: mask, **{q: np.zeros(w.shapes[q], bool) for q in held if q != p}})
            got = outs[p].cpu().numpy().view(np.uint32)
            assert (got[mask] == src[p].view(np.uint32)[mask]).all(), (r, p)
            assert (got[~mask] == sentinel).all(), (r, p)
        # bf16 fold widens exactly
        dst.fill_(float("nan"))
        fz.fp8z1_fold(t, d16, fz.BF16, dst)
        want16 = layout.fold_shard(tab, {p: layout.widen_bf16(src16[p]) for p in held})
        assert gh.bits_equal(gh.folded(dst, n), want16), (r, "bf16")
        t.free()


@pytest.mark.parametrize("name", ["moe_small", "ragged_small", "full_small", "wide_rows_small"])
def test_unfold_codes_at_any_destination_alignment(name):
    """FP8 unfold of random codes (padding bytes random too: they must be dropped) into
    destinations at byte offsets 0, 1, 16, 64 and 127 of a sentinel-filled buffer: the
    shard's real positions get the oracle's bytes, no other byte (inside the param or in
    the margins around it) changes; scales land in [E, Rb, Cb].  Covers both unfold
    kernels (by blocks when rows start on 128-byte lines, by rows otherwise), with
    rows up to 40,000 codes long."""
    gh = _gh()
    w = synth.get(name)
    rng = np.random.default_rng(17)
    for r in (0, w.dp - 1, otable.ALL_RANKS):
        tab = otable.build(w.shapes, w.dp, r)
        t = fz.fp8z1_build_table(w.shapes, w.dp, r)
        n = t.shard_slots
        held = gh.held_experts(tab["entries"])
        folded = rng.integers(0, 256, size=(n, 128, 128), dtype=np.uint8)
        fsc = rng.random(n).astype(np.float32)
        d_folded = torch.from_numpy(folded.reshape(-1)).cuda()
        d_fsc = torch.from_numpy(fsc).cuda()
        want = {p: np.zeros(s, np.uint8) for p, s in enumerate(w.shapes)}
        want_s = {p: np.zeros(otable.grid(s), np.float32) for p, s in enumerate(w.shapes)}
        layout.unfold_shard(tab, folded, want, fsc, want_s)
        mask = {p: np.zeros(s, bool) for p, s in enumerate(w.shapes)}
        layout.unfold_shard(tab, layout.valid_mask(tab), mask)
        for off in (0, 1, 16, 64, 127):
            bufs, outs, souts = {}, [], []
            for p, s in enumerate(w.shapes):
                if p not in held:
                    outs.append(None)
                    souts.append(None)
                    continue
                size = int(np.prod(s))
                bufs[p] = torch.full((size + 256,), 0xA5, dtype=torch.uint8, device="cuda")
                outs.append(bufs[p][off:off + size])
                souts.append(torch.full(otable.grid(s), float("nan"), dtype=torch.float32, device="cuda"))
            fz.fp8z1_unfold(t, d_folded, fz.E4M3, d_fsc, outs, souts)
            torch.cuda.synchronize()
            for p in held:
                b = bufs[p].cpu().numpy()
                size = int(np.prod(w.shapes[p]))
                assert (b[:off] == 0xA5).all() and (b[off + size:] == 0xA5).all(), (r, off, p, "margin")
                got = b[off:off + size].reshape(w.shapes[p])
                assert (got[mask[p]] == want[p][mask[p]]).all(), (r, off, p)
                assert (got[~mask[p]] == 0xA5).all(), (r, off, p, "outside the shard")
                blocks = np.zeros(otable.grid(w.shapes[p]), bool)
                for e in tab["entries"]:
                    if e["param"] == p:
                        blocks[int(e["expert"]), int(e["brow"]), int(e["bcol"])] = True
                gs = souts[p].cpu().numpy()
                assert gh.bits_equal(gs[blocks], want_s[p][blocks]), (r, off, p, "scales")
                assert np.isnan(gs[~blocks]).all(), (r, off, p, "scales outside the shard")
        t.free()


@pytest.mark.parametrize("name", ["tiny", "ragged_small", "moe_small"])
def test_fused_statistics_equal_separate_kernel(name):
    """Per-slot sums of squares written by the fold equal the separate statistics
    kernel's bit for bit, and the oracle's per-slot float64 sums to 1e-12."""
    gh = _gh()
    w = synth.get(name)
    hp = fz.Hparams.make(synth.Hparams(max_grad_norm=1.0))
    for r in range(min(w.dp, 4)):
        from blockwise_fp8_zero_fold_amd.shard import Shard
        sh = Shard(w.shapes, w.dp, r)
        tab = otable.build(w.shapes, w.dp, r)
        held = gh.held_experts(tab["entries"])
        g = gh.grad_tensors(w, held, 1)
        sh.init(hp, gh.master_tensors(w, held), fz.BF16 if w.master_dtype == "bf16" else fz.F32)
        sh.fold_grads(hp, g, fused_stats=True)
        fused = sh.workspace.cpu().numpy().copy()
        sh.update(hp, presummed=False)  # recomputes the sums with the statistics kernel
        sep = sh.workspace.cpu().numpy().copy()
        assert fused.tobytes() == sep.tobytes()
        sh.workspace.fill_(-1.0)
        sh.update_rowmajor(hp, g)  # the statistics pass over the row-major grads
        rowmajor = sh.workspace.cpu().numpy()
        assert fused.tobytes() == rowmajor.tobytes()
        gf = layout.fold_shard(tab, harness.grads(w, 1))
        mask = layout.valid_mask(tab)
        n = len(mask)
        parts = fused[:n * fz.STAT_PARTS].reshape(n, fz.STAT_PARTS)
        rows = 128 // fz.STAT_PARTS
        for q in range(fz.STAT_PARTS):
            sl = slice(rows * q, rows * (q + 1))
            want_q = np.array([optim.local_sumsq(gf[s][sl][mask[s][sl]]) for s in range(n)])
            assert np.all(np.abs(parts[:, q] - want_q) <= 1e-12 * np.abs(want_q)), q
        want = np.array([optim.local_sumsq(gf[s][mask[s]]) for s in range(n)])
        assert np.all(np.abs(parts.sum(axis=1) - want) <= 1e-12 * np.abs(want))


# ---------------------------------------------------------------- the step

def _bar(got, want, what):
    """The parity bar: float32 state within 1e-6 relative (with a floor of 1e-6*|lr| for
    values that cancel to near 0), exact equality expected."""
    g = got.astype(np.float64)
    x = want.astype(np.float64)
    both_nan = np.isnan(g) & np.isnan(x)
    ok = both_nan | (np.abs(g - x) <= 1e-6 * np.abs(x) + 1e-9)
    assert ok.all(), f"{what}: {int((~ok).sum())} elements outside 1e-6 relative"


def _codes_bar(got, want, what):
    if got.size == 0:  # a shard of padding slots only
        return
    d = oe4m3.ulp_distance(got, want)
    assert d.max() <= 1, f"{what}: code distance {d.max()}"
    assert (d > 0).mean() <= 1e-4, f"{what}: {(d > 0).mean()} of codes differ by 1 ulp"


def _run_parity(w, ranks=None, fused=None, fold_on_read=False):
    gh = _gh()
    from blockwise_fp8_zero_fold_amd.shard import Shard
    ranks = w.ranks if ranks is None else ranks
    ref, tabs = harness.run_sharded_all_ranks(w, ranks=ranks)
    un = harness.run_unsharded(w)
    split = fz.SPLIT_PARAM if w.split == "param" else fz.SPLIT_BLOCK
    dtype = fz.BF16 if w.master_dtype == "bf16" else fz.F32
    P0 = harness.masters(w)
    for r in ranks:
        tab = tabs[r]
        sh = Shard(w.shapes, w.dp, r, split)
        n = sh.n_slots
        held = gh.held_experts(tab["entries"])
        sh.init(fz.Hparams.make(w.hp), gh.master_tensors(w, held), dtype)
        assert gh.bits_equal(gh.folded(sh.master, n), layout.fold_shard(tab, P0)), "init fold"
        codes, scales = gh.code_tensors(w, held)
        mask = layout.valid_mask(tab)
        heldmask = {p: np.zeros(s, bool) for p, s in enumerate(w.shapes)}
        layout.unfold_shard(tab, mask, heldmask)
        blockmask = {p: np.zeros(otable.grid(s), bool) for p, s in enumerate(w.shapes)}
        for e in tab["entries"]:
            if e["param"] >= 0:
                blockmask[int(e["param"])][int(e["expert"]), int(e["brow"]), int(e["bcol"])] = True
        prev = harness.initial_reference(w, tab)
        rederived = False  # the reference chain left the precomputed one (a k that differed)
        for t in range(1, w.steps + 1):
            R = ref[r][t - 1]
            hp = fz.Hparams.make(w.hp, extra_sumsq=R["extra"])
            use_fused = (t % 2 == 0) if fused is None else fused
            sh.step(hp, gh.grad_tensors(w, held, t), codes, scales, fused_stats=use_fused, fold_on_read=fold_on_read)
            torch.cuda.synchronize()
            tag = f"{w.name} rank {r} step {t}" + (" (fold on read)" if fold_on_read else "")
            if not fold_on_read:
                assert gh.bits_equal(gh.folded(sh.grad, n), R["grad"]), f"{tag}: grad fold"
            st = sh.read_state()
            if rederived:
                R = harness.step_given_k(w, tab, prev, R["grad"], R["extra"], None)
            k_gpu = harness.clip_stage1(w.hp, prev["state"], st, R["state"], tag)
            if k_gpu is not None:  # stage 2: the oracle's step with the GPU's k
                print(f"# {tag}: k differs from the oracle's by the sum order; stage 2 with k={k_gpu!r}")
                R = harness.step_given_k(w, tab, prev, R["grad"], R["extra"], k_gpu)
                rederived = True
            prev = R
            want_st = R["state"]
            for key in ("step", "found_inf", "skipped_total", "good_steps"):
                assert st[key] == want_st[key], (tag, key, st[key], want_st[key])
            for key in ("k", "loss_scale", "step_size", "bc2_sqrt", "decay", "beta1_pow", "beta2_pow"):
                assert st[key] == want_st[key], (tag, key, st[key], want_st[key])
            for name, dt in (("master", np.float32), ("m", np.float32), ("v", np.float32)):
                got = gh.folded(getattr(sh, name), n)
                _bar(got[mask], R[name][mask], f"{tag}: {name}")
                assert gh.bits_equal(got, R[name]), f"{tag}: {name} not bit-exact {gh.first_diff(got, R[name])}"
            got_codes = gh.folded(sh.fp8, n, np.uint8)
            _codes_bar(got_codes[mask], R["codes"][mask], f"{tag}: codes")
            assert gh.bits_equal(got_codes, R["codes"]), f"{tag}: codes not bit-exact"
            got_sc = sh.scales.cpu().numpy()[:n]
            _bar(got_sc, R["scales"], f"{tag}: scales")
            assert gh.bits_equal(got_sc, R["scales"]), f"{tag}: scales not bit-exact"
            U = un[t - 1]
            if rederived and R["state"]["step"] > 0:
                # the unsharded run used the oracle's own k: unfold the re-derived shard instead
                U = dict(zip(("codes", "scales"), harness.unfold_all_ranks(w, {r: tab}, {r: R["codes"]}, np.uint8,
                                                                          scales={r: R["scales"]})))
            if U["codes"] is not None:
                for p in held:
                    c = codes[p].cpu().numpy()
                    assert (c[heldmask[p]] == U["codes"][p][heldmask[p]]).all(), f"{tag}: unfolded codes p{p}"
                    assert (c[~heldmask[p]] == 0xA5).all(), f"{tag}: unfold wrote outside the shard p{p}"
                    s = scales[p].cpu().numpy()
                    assert gh.bits_equal(s[blockmask[p]], U["scales"][p][blockmask[p]]), f"{tag}: scales p{p}"
                    assert np.isnan(s[~blockmask[p]]).all()


@pytest.mark.parametrize("name", ["tiny", "tiny_clip", "tiny_lossscale", "dense_small", "moe_small", "full_small",
                                  "lines_small", "tiny_pow2", "ragged_small_pow2"])
@pytest.mark.parametrize("fold_on_read", [False, True])
def test_step_parity(name, fold_on_read):
    _run_parity(synth.get(name), fold_on_read=fold_on_read)


@pytest.mark.parametrize("split", ["block", "param"])
@pytest.mark.parametrize("fold_on_read", [False, True])
def test_step_parity_ragged(split, fold_on_read):
    w = synth.get("ragged_small").with_(split=split)
    _run_parity(w, ranks=[0, 5, 7, 15], fold_on_read=fold_on_read)


def test_padding_poison_gpu():
    """NaN in the folded grad padding and NaN-payload sentinels in master/m/v padding:
    the step masks by the table, so no skip, sentinels unchanged, results as clean."""
    gh = _gh()
    from blockwise_fp8_zero_fold_amd.shard import Shard
    w = synth.get("tiny_clip")
    tab = otable.build(w.shapes, w.dp, 1)
    mask = torch.from_numpy(layout.valid_mask(tab).reshape(-1)).cuda()
    held = gh.held_experts(tab["entries"])
    hp = fz.Hparams.make(w.hp, extra_sumsq=0.0)
    res = []
    for poison in (False, True):
        sh = Shard(w.shapes, w.dp, 1)
        sh.init(hp, gh.master_tensors(w, held))
        sh.fold_grads(hp, gh.grad_tensors(w, held, 1), fused_stats=False)
        if poison:
            sent = torch.tensor([0x7FC0BEEF], dtype=torch.int32, device="cuda").view(torch.float32)
            sh.grad[~mask] = float("nan")
            for b in (sh.master, sh.m, sh.v):
                b[~mask] = sent
        sh.update(hp, presummed=False)
        torch.cuda.synchronize()
        res.append(sh)
    clean, dirty = res
    assert dirty.read_state()["found_inf"] == 0
    for name in ("master", "m", "v"):
        a, b = getattr(clean, name), getattr(dirty, name)
        assert torch.equal(a[mask].view(torch.int32), b[mask].view(torch.int32))
        assert bool((b[~mask].view(torch.int32) == 0x7FC0BEEF).all())
    assert torch.equal(clean.fp8, dirty.fp8) and torch.equal(clean.scales, dirty.scales)
    assert int(dirty.fp8[~mask].sum()) == 0


def test_determinism_and_resume():
    """Two runs give identical bits; 2 steps + save/restore + 3 steps equals 5 steps."""
    gh = _gh()
    from blockwise_fp8_zero_fold_amd.shard import Shard
    w = synth.get("tiny_lossscale")
    tab = otable.build(w.shapes, w.dp, 1)
    held = gh.held_experts(tab["entries"])
    hp = fz.Hparams.make(w.hp)
    grads = [gh.grad_tensors(w, held, t) for t in range(1, 6)]

    def run(steps, sh=None):
        if sh is None:
            sh = Shard(w.shapes, w.dp, 1)
            sh.init(hp, gh.master_tensors(w, held))
        codes, scales = gh.code_tensors(w, held)
        for t in steps:
            sh.step(hp, grads[t - 1], codes, scales)
        torch.cuda.synchronize()
        return sh

    a = run(range(1, 6))
    b = run(range(1, 6))
    for name in ("master", "m", "v", "fp8", "scales", "state"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    c = run(range(1, 3))
    saved = {name: getattr(c, name).clone() for name in ("master", "m", "v", "fp8", "scales")}
    st = c.read_state()
    d = Shard(w.shapes, w.dp, 1)
    for name, x in saved.items():
        getattr(d, name).copy_(x)
    fz.fp8z1_state_write(d.state, st)
    d = run(range(3, 6), d)
    for name in ("master", "m", "v", "fp8", "scales"):
        assert torch.equal(getattr(a, name), getattr(d, name)), name
    assert a.read_state() == d.read_state()


def test_empty_and_degenerate_blocks():
    """All-zero weights and grads (amax 0 -> scale 1, codes 0), a block of one element,
    and a 1x1 param."""
    gh = _gh()
    from blockwise_fp8_zero_fold_amd.shard import Shard
    w = synth.Workload(name="degen", shapes=((1, 1, 1), (1, 129, 1), (2, 1, 130)), dp=3, ranks=(0, 1, 2), steps=2,
                       hp=synth.Hparams(max_grad_norm=1.0), grad_sigma=0.0, master_sigma=0.0)
    _run_parity(w)
    _run_parity(w, fold_on_read=True)


@pytest.mark.parametrize("name,split", [("tiny", "block"), ("ragged_small", "block"), ("ragged_small", "param"),
                                        ("moe_small", "block"), ("dense_small", "block")])
def test_all_ranks_gather_and_whole_buffer_unfold(name, split):
    """Every rank steps its own shard; the ranks' folded FP8 codes and scales are
    concatenated in rank order (what the all-gathers produce) and unfolded with the
    table of the whole flat buffer.  The result equals the row-major definition."""
    gh = _gh()
    from blockwise_fp8_zero_fold_amd.shard import Shard
    w = synth.get(name).with_(split=split)
    steps = 2
    ref, tabs = harness.run_sharded_all_ranks(w, steps=steps)
    un = harness.run_unsharded(w, steps=steps)
    sid = fz.SPLIT_PARAM if split == "param" else fz.SPLIT_BLOCK
    dtype = fz.BF16 if w.master_dtype == "bf16" else fz.F32
    codes_all, scales_all = [], []
    for r in range(w.dp):
        sh = Shard(w.shapes, w.dp, r, sid)
        held = gh.held_experts(tabs[r]["entries"])
        sh.init(fz.Hparams.make(w.hp), gh.master_tensors(w, held), dtype)
        for t in range(1, steps + 1):
            hp = fz.Hparams.make(w.hp, extra_sumsq=ref[r][t - 1]["extra"])
            sh.update_rowmajor(hp, gh.grad_tensors(w, held, t))
        codes_all.append(sh.fp8[: sh.n_slots * 16384])
        scales_all.append(sh.scales[: sh.n_slots])
    gathered = torch.cat(codes_all)
    gscales = torch.cat(scales_all)
    whole = fz.fp8z1_build_table(w.shapes, w.dp, fz.ALL_RANKS, sid)
    assert whole.shard_slots * 16384 == gathered.numel()
    dst = [torch.full(s, 0xA5, dtype=torch.uint8, device="cuda") for s in w.shapes]
    dsc = [torch.full(otable.grid(s), float("nan"), dtype=torch.float32, device="cuda") for s in w.shapes]
    fz.fp8z1_unfold(whole, gathered, fz.E4M3, gscales, dst, dsc)
    torch.cuda.synchronize()
    U = un[steps - 1]
    for p in range(w.n_params):
        assert gh.bits_equal(dst[p].cpu().numpy(), U["codes"][p]), (name, split, p)
        assert gh.bits_equal(dsc[p].cpu().numpy(), U["scales"][p]), (name, split, p)


@pytest.mark.parametrize("shape", [(2, 200, 300), (3, 130, 400)])
def test_dequantize_every_code(shape):
    """All 256 codes times random scales (one per 128x128 block): float32 bit-exact
    against the oracle, bfloat16 equal to torch's RNE cast of the oracle's float32.
    C = 300 takes the any-alignment kernel, C = 400 the 16-code vector kernel."""
    from oracle import quant as oquant
    rng = np.random.default_rng(17)
    codes = rng.integers(0, 256, size=shape, dtype=np.uint8)
    codes[0, 0, :256] = np.arange(256, dtype=np.uint8)
    scales = (2.0 ** rng.uniform(-20, 20, size=otable.grid(shape))).astype(np.float32)
    want = oquant.dequantize(codes, scales)
    dc, ds = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
    out = torch.empty(shape, dtype=torch.float32, device="cuda")
    fz.fp8z1_dequantize(dc, ds, shape, fz.F32, out)
    got = out.cpu().numpy()
    nan = np.isnan(want)
    assert (np.isnan(got) == nan).all()
    assert got[~nan].tobytes() == want[~nan].tobytes()
    ob = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    fz.fp8z1_dequantize(dc, ds, shape, fz.BF16, ob)
    gb = ob.float().cpu().numpy()
    wb = torch.from_numpy(want).to(torch.bfloat16).float().numpy()
    assert (np.isnan(gb) == nan).all()
    assert gb[~nan].tobytes() == wb[~nan].tobytes()


@pytest.mark.parametrize("shape", [(1, 256, 2048), (1, 130, 300)])
def test_dequantize_extreme_scales(shape):
    """Every code times block scales at the ends of the float32 range: products that
    are subnormal or round to zero, scales that are subnormal themselves, products
    that overflow to infinity (and, in BF16, finite floats that round up to it).
    Float32 bit-exact against the oracle, bfloat16 equal to torch's RNE cast of it;
    C = 2048 takes the vector kernel, C = 300 the any-alignment one."""
    from oracle import quant as oquant
    codes = (np.arange(int(np.prod(shape))) % 256).astype(np.uint8).reshape(shape)
    picks = np.array([2.0 ** -149, 2.0 ** -140, 2.0 ** -130, 2.0 ** -127, 2.0 ** -126, 1.1754942e-38 * 0.75,
                      1e-30, 2.0 ** -9, 1.0 / 448, 1.0, 3.0, 2.0 ** 100, 2.0 ** 119, 1e36, 3.0e38,
                      float(np.finfo(np.float32).max)], dtype=np.float64).astype(np.float32)
    g = otable.grid(shape)
    scales = picks[(5 * np.arange(int(np.prod(g)))) % len(picks)].reshape(g)  # both ends in any grid
    want = oquant.dequantize(codes, scales)
    assert np.isinf(want).any() and (want[np.isfinite(want)] != 0).any()
    tiny = np.abs(want[np.isfinite(want)])
    assert ((tiny > 0) & (tiny < np.finfo(np.float32).tiny)).any(), "some products must be subnormal"
    dc, ds = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
    out = torch.empty(shape, dtype=torch.float32, device="cuda")
    fz.fp8z1_dequantize(dc, ds, shape, fz.F32, out)
    got = out.cpu().numpy()
    nan = np.isnan(want)
    assert (np.isnan(got) == nan).all()
    assert got[~nan].tobytes() == want[~nan].tobytes()
    ob = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    fz.fp8z1_dequantize(dc, ds, shape, fz.BF16, ob)
    gb = ob.float().cpu().numpy()
    wb = torch.from_numpy(want).to(torch.bfloat16).float().numpy()
    assert (np.isnan(gb) == nan).all()
    assert gb[~nan].tobytes() == wb[~nan].tobytes()


@pytest.mark.parametrize("name", ["moe_small", "full_small"])
def test_dequantized_weights_track_the_master(name):
    """After a few steps the dequantized FP8 weights stay close to the FP32 master:
    cosine > 0.995 per block and under 0.5% of real elements quantized to zero
    (the health thresholds of the quantization-error table of the FP8-training page)."""
    gh = _gh()
    from blockwise_fp8_zero_fold_amd.shard import Shard
    w = synth.get(name)
    dtype = fz.BF16 if w.master_dtype == "bf16" else fz.F32
    ref, tabs = harness.run_sharded_all_ranks(w, ranks=[0])
    tab = tabs[0]
    held = gh.held_experts(tab["entries"])
    sh = Shard(w.shapes, w.dp, 0)
    sh.init(fz.Hparams.make(w.hp), gh.master_tensors(w, held), dtype)
    codes, scales = gh.code_tensors(w, held)
    for t in range(1, w.steps + 1):
        sh.step(fz.Hparams.make(w.hp, extra_sumsq=ref[0][t - 1]["extra"]), gh.grad_tensors(w, held, t), codes, scales,
                fold_on_read=True)
    masters = [torch.full(s, float("nan"), dtype=torch.float32, device="cuda") if p in held else None
               for p, s in enumerate(w.shapes)]
    fz.fp8z1_unfold(sh.table, sh.master, fz.F32, None, masters)
    zeros = total = 0
    worst = 1.0
    for p in held:
        deq = torch.empty(w.shapes[p], dtype=torch.float32, device="cuda")
        fz.fp8z1_dequantize(codes[p], scales[p], w.shapes[p], fz.F32, deq)
        mask = torch.from_numpy(np.isin(np.arange(w.shapes[p][0]), held[p])).cuda()
        a, b = deq[mask].double(), masters[p][mask].double()
        E, R, C = a.shape
        for br in range(0, R, 128):
            for bc in range(0, C, 128):
                x, y = a[:, br:br + 128, bc:bc + 128], b[:, br:br + 128, bc:bc + 128]
                cos = (x * y).sum(dim=(1, 2)) / (x.norm(dim=(1, 2)) * y.norm(dim=(1, 2)))
                worst = min(worst, float(cos.min()))
        zeros += int((codes[p][mask] & 0x7F).eq(0).sum())
        total += a.numel()
    assert worst > 0.995, worst
    assert zeros / total < 0.005, zeros / total


def test_extreme_shapes_and_all_padding_ranks():
    """Widest and tallest params the 16-bit block indices allow (65,536 block columns /
    rows, one real row / column per block), and more ranks than blocks (ranks whose
    shard is all padding slots)."""
    wide = synth.Workload(name="extreme", shapes=((1, 1, (1 << 23) - 1), (1, (1 << 23) - 1, 1)), dp=64,
                          ranks=(0, 31, 63), steps=1, hp=synth.Hparams(max_grad_norm=1.0), grad_sigma=1e-3)
    tabs = {r: otable.build(wide.shapes, wide.dp, r) for r in wide.ranks}
    ent = np.concatenate([tabs[r]["entries"] for r in wide.ranks])
    assert ent["bcol"].max() == 65535 and ent["brow"].max() == 65535
    assert ent["vcols"].min() == 1 and ent["vrows"].min() == 1
    _run_parity(wide)
    _run_parity(wide, fold_on_read=True)
    few = synth.Workload(name="few_blocks", shapes=((1, 130, 70),), dp=16, ranks=(0, 1, 2, 15), steps=2,
                         hp=synth.Hparams(max_grad_norm=1.0), grad_sigma=1e-3)
    assert (otable.build(few.shapes, few.dp, 15)["entries"]["param"] < 0).all()
    _run_parity(few)
    _run_parity(few, fold_on_read=True)


def test_thirty_steps_of_loss_scaling_and_clipping():
    """30 steps: the loss scale doubles every 2 clean steps and halves on the injected
    overflow, clipping stays active; every rank's state and folded buffers stay equal
    to the oracle's bit for bit after every step, on both routes."""
    w = synth.get("tiny_lossscale").with_(name="tiny_lossscale_30", steps=30)
    _run_parity(w)
    _run_parity(w, fold_on_read=True)


@pytest.mark.parametrize("seed", range(8))
def test_random_shape_sets(seed):
    """Random sets of 1-5 params (E 1-3, R and C 1-400, so most rows start off any
    alignment), random DP, split, clipping / loss scaling and scale rule: the whole step
    on both routes, every rank listed, bit for bit against the oracle."""
    rng = np.random.default_rng(1000 + seed)
    k = int(rng.integers(1, 6))
    shapes = tuple((int(rng.integers(1, 4)), int(rng.integers(1, 401)), int(rng.integers(1, 401))) for _ in range(k))
    dp = int(rng.integers(1, 7))
    hp = synth.Hparams(max_grad_norm=float(rng.choice([0.0, 0.05, 1.0])), loss_scaling=bool(rng.integers(0, 2)),
                       init_scale=256.0, growth_interval=1, scale_rule=int(rng.integers(0, 2)))
    w = synth.Workload(name=f"random{seed}", shapes=shapes, dp=dp, ranks=tuple(range(dp)), steps=2, hp=hp,
                       split=str(rng.choice(["block", "param"])), grad_sigma=1e-3,
                       grad_premult=256.0 if hp.loss_scaling else 1.0)
    print(f"# {w.name}: shapes {shapes} dp {dp} split {w.split} hp {hp}", flush=True)
    _run_parity(w)
    _run_parity(w, fold_on_read=True)


@pytest.mark.parametrize("seed", range(6))
def test_random_hyperparameters(seed):
    """AdamW and loss-scale settings away from the usual ones: learning rates from
    1e-5 to 0.3, beta1 and beta2 down to 0 and up to 0.9999, eps from 1e-12 to 1e-3,
    weight decay from 0 to 1, growth and backoff factors other than 2 and 0.5, over
    five steps on both routes and every rank, bit for bit against the oracle."""
    rng = np.random.default_rng(2000 + seed)
    pick = lambda xs: float(rng.choice(xs))
    hp = synth.Hparams(lr=float(10.0 ** rng.uniform(-5, np.log10(0.3))), beta1=pick([0.0, 0.5, 0.9, 0.99]),
                       beta2=pick([0.0, 0.9, 0.999, 0.9999]), eps=pick([1e-12, 1e-8, 1e-3]),
                       weight_decay=pick([0.0, 0.01, 0.1, 1.0]), max_grad_norm=pick([0.0, 0.01, 1.0]),
                       loss_scaling=bool(rng.integers(0, 2)), init_scale=pick([1.0, 256.0, 2.0 ** 20]),
                       growth_factor=pick([1.5, 2.0, 4.0]), backoff_factor=pick([0.25, 0.5, 0.75]),
                       growth_interval=int(rng.integers(1, 4)), scale_rule=int(rng.integers(0, 2)))
    w = synth.Workload(name=f"hparams{seed}", shapes=((2, 200, 300), (1, 256, 128)), dp=2, ranks=(0, 1), steps=5,
                       hp=hp, grad_sigma=1e-3, grad_premult=hp.init_scale if hp.loss_scaling else 1.0,
                       inf_block=(3, 0, 1, 1, 2) if seed % 2 else None)
    print(f"# {w.name}: {hp}", flush=True)
    _run_parity(w)
    _run_parity(w, fold_on_read=True)


@pytest.mark.parametrize("name,rank,mode", [("tiny_clip", 1, "eager"), ("full_small", 0, "graph")])
def test_c_abi_consumer_without_python(tmp_path, name, rank, mode):
    """A C++ program (tests/native/abi_c_step.cpp, built with the library) drives the
    ABI with its own HIP allocations and stream, no torch in the process; its outputs
    equal the oracle's.  "graph": the statistics go through fp8z1_shard_sumsq and
    hp.d_global_sumsq, and steps 2.. are launches of one captured HIP graph (the
    full_small set: clipping, loss scaling and a skipped step among the replays)."""
    import subprocess
    exe = os.path.join(os.path.dirname(__file__), "native", "abi_c_step")
    if not os.path.exists(exe):
        pytest.fail("tests/native/abi_c_step is not built (blockwise_fp8_zero_fold_amd/build.py builds it)")
    w = synth.get(name)
    ref, tabs = harness.run_sharded_all_ranks(w, ranks=[rank])
    un = harness.run_unsharded(w)
    P = harness.masters(w)
    hp = w.hp
    with open(tmp_path / "meta.txt", "w") as f:
        f.write(f"{w.n_params} {w.dp} {rank} {w.steps}\n")
        for e, r, c in w.shapes:
            f.write(f"{e} {r} {c}\n")
        f32 = [repr(float(np.float32(x))) for x in (hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay,
                                                     hp.max_grad_norm)]  # exact float32 values
        f.write(" ".join(f32) + "\n")
        f.write(f"{int(hp.loss_scaling)} {float(np.float32(hp.init_scale))!r} {float(np.float32(hp.growth_factor))!r} "
                f"{float(np.float32(hp.backoff_factor))!r} {int(hp.growth_interval)} {int(hp.scale_rule)}\n")
        for t in range(w.steps):
            f.write(f"{ref[rank][t]['extra']!r}\n")
    if mode == "graph":
        assert w.dp == 1 and all(ref[rank][t]["extra"] == 0 for t in range(w.steps))
        assert any(ref[rank][t]["state"]["found_inf"] for t in range(1, w.steps))
    for p in range(w.n_params):
        P[p].tofile(tmp_path / f"master_{p}.bin")
    for t in range(1, w.steps + 1):
        G = harness.grads(w, t)
        for p in range(w.n_params):
            G[p].tofile(tmp_path / f"grad_{t}_{p}.bin")
    env = {k: v for k, v in os.environ.items() if k != "PYTHONPATH"}
    args = [exe, str(tmp_path)] + (["graph"] if mode == "graph" else [])
    r = subprocess.run(args, capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stderr
    R = ref[rank][-1]
    n = tabs[rank]["shard_slots"]
    got = np.fromfile(tmp_path / "out_master.bin", dtype=np.float32).reshape(n, 128, 128)
    assert got.tobytes() == R["master"].tobytes()
    step, k, found, skipped = open(tmp_path / "out_state.txt").read().split()
    assert int(step) == R["state"]["step"] and float(k) == R["state"]["k"]
    assert int(found) == R["state"]["found_inf"] and int(skipped) == R["state"]["skipped_total"]
    mask = layout.valid_mask(tabs[rank])
    held = {p: np.zeros(s, bool) for p, s in enumerate(w.shapes)}
    layout.unfold_shard(tabs[rank], mask, held)
    for p in range(w.n_params):
        codes = np.fromfile(tmp_path / f"out_codes_{p}.bin", dtype=np.uint8).reshape(w.shapes[p])
        assert (codes[held[p]] == un[-1]["codes"][p][held[p]]).all()
        blocks = np.zeros(otable.grid(w.shapes[p]), bool)
        for e in tabs[rank]["entries"]:
            if e["param"] == p:
                blocks[int(e["expert"]), int(e["brow"]), int(e["bcol"])] = True
        sc = np.fromfile(tmp_path / f"out_scales_{p}.bin", dtype=np.float32).reshape(otable.grid(w.shapes[p]))
        assert sc[blocks].tobytes() == un[-1]["scales"][p][blocks].tobytes()
