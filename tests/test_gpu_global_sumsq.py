"""GPU: every rank of a DP group run on the one GPU, with the statistics reduced on the
device: each rank's fold (or statistics-only pass) writes its partials,
fp8z1_shard_sumsq sums them into one double per rank, a device-side sum of those
stands in for the all-reduce, and every rank's step reads the result through
hp.d_global_sumsq.  Each rank's results are checked bit for bit against the oracle,
including a step skipped because one rank's grads hold an inf."""
import numpy as np
import pytest

import synth
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


@pytest.mark.parametrize("name", ["dense_small", "tiny_lossscale"])
@pytest.mark.parametrize("fold_on_read", [True, False])
def test_device_reduced_statistics_equal_oracle(name, fold_on_read):
    from tests import gpu_harness as gh
    from blockwise_fp8_zero_fold_amd.shard import Shard
    w = synth.get(name)
    ranks = list(range(w.dp))
    ref, tabs = harness.run_sharded_all_ranks(w, ranks=ranks)
    sh, held, codes, scales = {}, {}, {}, {}
    hp0 = fz.Hparams.make(w.hp)
    for r in ranks:
        sh[r] = Shard(w.shapes, w.dp, r)
        held[r] = gh.held_experts(tabs[r]["entries"])
        sh[r].init(hp0, gh.master_tensors(w, held[r]), fz.F32)
        codes[r], scales[r] = gh.code_tensors(w, held[r])
    sums = torch.zeros(w.dp, dtype=torch.float64, device="cuda")
    glob = torch.zeros(1, dtype=torch.float64, device="cuda")
    hp = fz.Hparams.make(w.hp, global_sumsq=glob)
    masks = {r: layout.valid_mask(tabs[r]) for r in ranks}
    for t in range(1, w.steps + 1):
        tag = f"{name} fold_on_read={fold_on_read} step {t}"
        print(f"# {tag}", flush=True)
        grads = {r: gh.grad_tensors(w, held[r], t) for r in ranks}
        for r in ranks:
            s = sh[r]
            dst = None if fold_on_read else s.grad
            fz.fp8z1_fold(s.table, grads[r], fz.F32, dst, slot_sumsq=s.workspace)
            fz.fp8z1_shard_sumsq(s.table, s.workspace, sums[r:r + 1])
        glob.copy_(sums.sum().reshape(1))  # stands in for the all-reduce
        for r in ranks:
            s = sh[r]
            if fold_on_read:
                fz.fp8z1_step_rowmajor(s.table, hp, s.state, grads[r], s.master, s.m, s.v, s.fp8, s.scales)
            else:
                fz.fp8z1_step(s.table, hp, s.state, s.grad, s.master, s.m, s.v, s.fp8, s.scales)
            s.unfold(codes[r], scales[r])
        torch.cuda.synchronize()
        got_sums = sums.cpu().numpy()
        for r in ranks:
            R = ref[r][t - 1]
            want_local = optim.local_sumsq(R["grad"][masks[r]])
            a = got_sums[r]
            assert (np.isinf(a) and np.isinf(want_local)) or abs(a - want_local) <= 1e-12 * abs(want_local), \
                (tag, r, a, want_local)
            n = sh[r].n_slots
            st = sh[r].read_state()
            for key in ("step", "found_inf", "skipped_total", "good_steps", "k", "loss_scale", "step_size"):
                assert st[key] == R["state"][key], (tag, r, key, st[key], R["state"][key])
            a, b = st["global_sumsq"], R["state"]["global_sumsq"]
            assert (np.isinf(a) and np.isinf(b)) or abs(a - b) <= 1e-12 * abs(b), (tag, r, a, b)
            for key in ("master", "m", "v"):
                assert gh.bits_equal(gh.folded(getattr(sh[r], key), n), R[key]), f"{tag}: rank {r} {key}"
            assert gh.bits_equal(gh.folded(sh[r].fp8, n, np.uint8), R["codes"]), f"{tag}: rank {r} codes"
            assert gh.bits_equal(sh[r].scales.cpu().numpy()[:n], R["scales"]), f"{tag}: rank {r} scales"
    if name == "tiny_lossscale":
        assert any(ref[0][t]["state"]["found_inf"] for t in range(w.steps)), "the inf step must be covered"
    # every rank's unfolded codes together give the whole row-major FP8 weights
    un = harness.run_unsharded(w)[w.steps - 1]
    whole = {p: np.full(s, 0xA5, np.uint8) for p, s in enumerate(w.shapes)}
    for r in ranks:
        m = {p: np.zeros(s, bool) for p, s in enumerate(w.shapes)}
        layout.unfold_shard(otable.build(w.shapes, w.dp, r), masks[r], m)
        for p in held[r]:
            whole[p][m[p]] = codes[r][p].cpu().numpy()[m[p]]
    for p in range(len(w.shapes)):
        assert gh.bits_equal(whole[p], un["codes"][p]), f"{name}: whole unfolded codes p{p}"
