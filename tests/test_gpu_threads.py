"""GPU: calls on distinct tables from several host threads at once, each thread on its
own stream (the binding releases the interpreter lock during library calls, so the
calls really overlap).  Each rank's results equal the oracle's bit for bit."""
import threading

import numpy as np
import pytest

import synth
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


@pytest.mark.parametrize("fold_on_read", [True, False])
def test_ranks_stepped_from_concurrent_threads(fold_on_read):
    from tests import gpu_harness as gh
    from blockwise_fp8_zero_fold_amd.shard import Shard
    w = synth.get("dense_small")  # DP = 8, clipping: the ranks share the global norm through extra_sumsq
    ref, tabs = harness.run_sharded_all_ranks(w)
    results, errors = {}, []

    def run(r):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                held = gh.held_experts(tabs[r]["entries"])
                sh = Shard(w.shapes, w.dp, r)
                sh.init(fz.Hparams.make(w.hp), gh.master_tensors(w, held), fz.F32)
                codes, scales = gh.code_tensors(w, held)
                for t in range(1, w.steps + 1):
                    hp = fz.Hparams.make(w.hp, extra_sumsq=ref[r][t - 1]["extra"])
                    sh.step(hp, gh.grad_tensors(w, held, t), codes, scales, fold_on_read=fold_on_read)
                s.synchronize()
                n = sh.n_slots
                results[r] = (sh.read_state(), gh.folded(sh.master, n), gh.folded(sh.fp8, n, np.uint8),
                              sh.scales.cpu().numpy()[:n])
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append((r, repr(e)))

    threads = [threading.Thread(target=run, args=(r,)) for r in range(w.dp)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for r in range(w.dp):
        R = ref[r][-1]
        st, master, codes, scales = results[r]
        assert st["step"] == R["state"]["step"] and st["k"] == R["state"]["k"], r
        assert gh.bits_equal(master, R["master"]), r
        assert gh.bits_equal(codes, R["codes"]), r
        assert gh.bits_equal(scales, R["scales"]), r
