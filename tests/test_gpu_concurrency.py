"""GPU: calls on distinct tables are independent and may run at the same time.  Two
shards with different tables (shapes, split, settings) are stepped concurrently from
two host threads, each on its own stream (default priority), and every result is bit
for bit the one the same shard gives when stepped alone on the default stream."""
import threading

import numpy as np
import pytest

import synth
from oracle import table as otable

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

fz = None


def setup_module(module):
    global fz
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import blockwise_fp8_zero_fold_amd as _fz  # raises if the library is not built
    fz = _fz


CASES = (("tiny_lossscale", 1, "block"), ("ragged_small", 5, "param"))
STEPS = 4


def _prepare(name, rank, split):
    from tests import gpu_harness as gh
    from blockwise_fp8_zero_fold_amd.shard import Shard
    w = synth.get(name).with_(split=split)
    tab = otable.build(w.shapes, w.dp, rank, otable.PARAM if split == "param" else otable.BLOCK)
    held = gh.held_experts(tab["entries"])
    sh = Shard(w.shapes, w.dp, rank, fz.SPLIT_PARAM if split == "param" else fz.SPLIT_BLOCK)
    hp = fz.Hparams.make(w.hp, extra_sumsq=0.0)
    masters = gh.master_tensors(w, held)
    grads = [gh.grad_tensors(w, held, t) for t in range(1, STEPS + 1)]
    codes, scales = gh.code_tensors(w, held)
    return dict(w=w, sh=sh, hp=hp, masters=masters, grads=grads, codes=codes, scales=scales,
                dtype=fz.BF16 if w.master_dtype == "bf16" else fz.F32)


def _run(c, stream=None):
    ctx = torch.cuda.stream(stream) if stream is not None else torch.cuda.stream(torch.cuda.current_stream())
    with ctx:
        sh = c["sh"]
        sh.init(c["hp"], c["masters"], c["dtype"])
        for t in range(STEPS):
            sh.step(c["hp"], c["grads"][t], c["codes"], c["scales"], fold_on_read=t % 2 == 1)
        c["state"] = sh.read_state()  # synchronizes this stream


def _results(c):
    sh = c["sh"]
    out = {name: getattr(sh, name).cpu().numpy().copy() for name in ("master", "m", "v", "fp8", "scales")}
    for p, (x, y) in enumerate(zip(c["codes"], c["scales"])):
        if x is not None:
            out[f"codes{p}"] = x.cpu().numpy().copy()
            out[f"scales{p}"] = y.cpu().numpy().copy()
    return out


def test_two_tables_stepped_from_two_threads_on_two_streams():
    alone = []
    for case in CASES:
        c = _prepare(*case)
        torch.cuda.synchronize()
        _run(c)
        torch.cuda.synchronize()
        alone.append((c["state"], _results(c)))
    together = [_prepare(*case) for case in CASES]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in CASES]  # default priority
    errors = []

    def worker(c, s):
        try:
            _run(c, s)
        except Exception as e:  # reported below, after both threads end
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(c, s)) for c, s in zip(together, streams)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    torch.cuda.synchronize()
    assert not errors, errors
    assert all(not th.is_alive() for th in threads)
    for case, (st, res), c in zip(CASES, alone, together):
        assert c["state"] == st, case
        got = _results(c)
        for key, want in res.items():
            assert got[key].tobytes() == want.tobytes(), (case, key)
