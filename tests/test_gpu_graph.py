"""GPU: the whole shard step captured once into a HIP graph and replayed, step after
step, with new grads copied into the captured grad buffers between replays.  Every
replay is checked bit for bit against the oracle (state, folded master/m/v/codes/
scales, unfolded codes and scales), with eager work and synchronizations between
replays.  Also: set-up work that cannot be captured is refused before any launch."""
import numpy as np
import pytest

import synth
from oracle import layout, table as otable
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


def _check(gh, sh, tab, R, U, held, codes, scales, tag):
    n = sh.n_slots
    st = sh.read_state()
    for key in ("step", "found_inf", "skipped_total", "good_steps", "k", "loss_scale", "step_size", "bc2_sqrt",
                "decay", "beta1_pow", "beta2_pow"):
        assert st[key] == R["state"][key], (tag, key, st[key], R["state"][key])
    a, b = st["global_sumsq"], R["state"]["global_sumsq"]
    assert (np.isinf(a) and np.isinf(b)) or abs(a - b) <= 1e-12 * abs(b), (tag, a, b)
    for name in ("master", "m", "v"):
        assert gh.bits_equal(gh.folded(getattr(sh, name), n), R[name]), f"{tag}: {name}"
    assert gh.bits_equal(gh.folded(sh.fp8, n, np.uint8), R["codes"]), f"{tag}: codes"
    assert gh.bits_equal(sh.scales.cpu().numpy()[:n], R["scales"]), f"{tag}: scales"
    heldmask = {p: np.zeros(s, bool) for p, s in enumerate(sh.shapes)}
    layout.unfold_shard(tab, layout.valid_mask(tab), heldmask)
    for p in held:
        c = codes[p].cpu().numpy()
        assert (c[heldmask[p]] == U["codes"][p][heldmask[p]]).all(), f"{tag}: unfolded codes p{p}"
        got_s, want_s = scales[p].cpu().numpy(), U["scales"][p]
        blocks = np.zeros(otable.grid(sh.shapes[p]), bool)
        for e in tab["entries"]:
            if e["param"] == p:
                blocks[int(e["expert"]), int(e["brow"]), int(e["bcol"])] = True
        assert gh.bits_equal(got_s[blocks], want_s[blocks]), f"{tag}: unfolded scales p{p}"


@pytest.mark.parametrize("fold_on_read,fused", [(True, True), (False, True), (False, False)])
def test_captured_step_replays_equal_oracle(fold_on_read, fused):
    """full_small: clipping + loss scaling, an inf grad at step 3 (a skipped step inside a
    replay), BF16 weights folded at init; one rank of DP = 1."""
    from tests import gpu_harness as gh
    from blockwise_fp8_zero_fold_amd.shard import Shard
    w = synth.get("full_small")
    ref, tabs = harness.run_sharded_all_ranks(w, ranks=[0])
    un = harness.run_unsharded(w)
    tab = tabs[0]
    held = gh.held_experts(tab["entries"])
    sh = Shard(w.shapes, w.dp, 0)
    hp = fz.Hparams.make(w.hp)
    sh.init(hp, gh.master_tensors(w, held), fz.BF16)
    codes, scales = gh.code_tensors(w, held)
    grads = gh.grad_tensors(w, held, 1)  # the captured grad buffers

    def run():
        sh.step(hp, grads, codes, scales, fused_stats=fused, fold_on_read=fold_on_read)

    tag = f"graph fold_on_read={fold_on_read} fused={fused}"
    print(f"# {tag}: eager step 1", flush=True)
    run()  # sets the table up on the device and uploads these pointer lists
    torch.cuda.synchronize()
    _check(gh, sh, tab, ref[0][0], un[0], held, codes, scales, f"{tag} step 1 (eager)")

    heldmask = {p: np.zeros(s, bool) for p, s in enumerate(w.shapes)}
    layout.unfold_shard(tab, layout.valid_mask(tab), heldmask)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    # capturing launched nothing: the state is still the one after step 1
    assert sh.read_state()["step"] == ref[0][0]["state"]["step"]
    for t in range(2, w.steps + 1):
        print(f"# {tag}: replay for step {t}", flush=True)
        new = gh.grad_tensors(w, held, t)
        for dst, src in zip(grads, new):
            if dst is not None:
                dst.copy_(src)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _check(gh, sh, tab, ref[0][t - 1], un[t - 1], held, codes, scales, f"{tag} step {t} (replay)")
        if t > 2:  # the FP32 read-back of the previous replay must not have been written over
            for p in held:
                assert gh.bits_equal(readback[p].cpu().numpy()[heldmask[p]], want_rb[p][heldmask[p]]), (tag, t, p)
        # an uncaptured FP32 unfold of the master into new arrays between replays: it has
        # its own pointer list, so the next replay still writes codes where it was captured to
        readback = [torch.zeros(s, dtype=torch.float32, device="cuda") if p in held else None
                    for p, s in enumerate(w.shapes)]
        fz.fp8z1_unfold(sh.table, sh.master, fz.F32, None, readback)
        torch.cuda.synchronize()
        want_rb = {p: np.zeros(s, np.float32) for p, s in enumerate(w.shapes)}
        layout.unfold_shard(tab, ref[0][t - 1]["master"], want_rb)
        for p in held:
            assert gh.bits_equal(readback[p].cpu().numpy()[heldmask[p]], want_rb[p][heldmask[p]]), (tag, t, p)
    assert any(r["state"]["found_inf"] for r in ref[0][1:]), "a skipped step must be among the replays"
    del g


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")  # the refused captures launch nothing
def test_capture_refuses_set_up_work():
    """A first device use of a table, or param pointers that differ from the last call,
    inside a capture: the call fails with a clear error before launching anything.  The
    same call with the pointers of the last uncaptured call captures, and its replays
    reproduce the uncaptured result."""
    from tests import gpu_harness as gh
    from blockwise_fp8_zero_fold_amd.shard import Shard
    w = synth.get("tiny_clip")
    held = gh.held_experts(otable.build(w.shapes, w.dp, 1)["entries"])
    hp = fz.Hparams.make(w.hp, extra_sumsq=0.0)
    sh = Shard(w.shapes, w.dp, 1)
    masters = gh.master_tensors(w, held)
    g = torch.cuda.CUDAGraph()
    with pytest.raises(fz.Fp8z1Error, match="stream capture"):
        with torch.cuda.graph(g):
            sh.init(hp, masters, fz.F32)  # first device use of this table
    torch.cuda.synchronize()
    sh.init(hp, masters, fz.F32)
    codes, scales = gh.code_tensors(w, held)
    sh.step(hp, gh.grad_tensors(w, held, 1), codes, scales)
    torch.cuda.synchronize()
    want_c = {p: codes[p].cpu().numpy().copy() for p in held}
    want_s = {p: scales[p].cpu().numpy().copy() for p in held}
    other_codes, other_scales = gh.code_tensors(w, held)
    g2 = torch.cuda.CUDAGraph()
    with pytest.raises(fz.Fp8z1Error, match="stream capture"):
        with torch.cuda.graph(g2):
            sh.unfold(other_codes, other_scales)  # new destination pointers
    torch.cuda.synchronize()
    g3 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g3):
        sh.unfold(codes, scales)
    for i in range(3):
        for p in held:
            codes[p].fill_(0xA5)
            scales[p].fill_(float("nan"))
        torch.cuda.synchronize()
        g3.replay()
        torch.cuda.synchronize()
        for p in held:
            assert gh.bits_equal(codes[p].cpu().numpy(), want_c[p]), (i, p)
            assert gh.bits_equal(scales[p].cpu().numpy(), want_s[p]), (i, p)
