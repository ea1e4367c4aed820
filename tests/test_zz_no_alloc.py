"""GPU: fp8z1_step_rowmajor_noalloc (the step that allocates nothing, its statistics
partials in the library's own device array) against fp8z1_step_rowmajor with a
caller workspace, through the C-ABI, on identical copies of the inputs: state,
master, m, v, codes and scales bit for bit.  Two calls in a row on the one array,
the second on a smaller shard (the array then holds the first call's larger
partials), with clipping on so that the partials are used; the first call with loss
scaling and an inf grad (a skipped step).  Also the refusals: a table not yet set
up on the device, a table beyond the size limit."""
import numpy as np
import pytest

import synth
from oracle import table as otable

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _fz():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import blockwise_fp8_zero_fold_amd as fz
    return fz


def _pair(fz, w, rank, steps, extra):
    """Two shards of the same rank with identical inputs; one stepped by the workspace
    entry point, the other by the no-alloc one; both compared after every step."""
    from blockwise_fp8_zero_fold_amd.shard import Shard
    from tests import gpu_harness as gh

    tab = otable.build(w.shapes, w.dp, rank, otable.BLOCK)
    held = gh.held_experts(tab["entries"])
    masters = gh.master_tensors(w, held)
    dtype = fz.BF16 if w.master_dtype == "bf16" else fz.F32
    a, b = Shard(w.shapes, w.dp, rank), Shard(w.shapes, w.dp, rank)
    for sh in (a, b):
        sh.init(fz.Hparams.make(w.hp), masters, dtype)  # sets the tables up on the device
    n = a.n_slots
    for t in range(1, steps + 1):
        hp = fz.Hparams.make(w.hp, extra_sumsq=extra)
        grads = gh.grad_tensors(w, held, t)
        a.update_rowmajor(hp, grads)
        fz.fp8z1_step_rowmajor_noalloc(b.table, hp, b.state, grads, b.master, b.m, b.v, b.fp8, b.scales)
        torch.cuda.synchronize()
        tag = f"{w.name} rank {rank} step {t}"
        sa, sb = a.read_state(), b.read_state()
        assert sa == sb, (tag, sa, sb)
        for name in ("master", "m", "v"):
            assert gh.bits_equal(gh.folded(getattr(a, name), n), gh.folded(getattr(b, name), n)), f"{tag}: {name}"
        assert gh.bits_equal(gh.folded(a.fp8, n, np.uint8), gh.folded(b.fp8, n, np.uint8)), f"{tag}: codes"
        assert gh.bits_equal(a.scales.cpu().numpy()[:n], b.scales.cpu().numpy()[:n]), f"{tag}: scales"
    return sa


def test_noalloc_step_equals_workspace_step():
    """full_small (60 slots: clipping, loss scaling, an inf grad that skips step 3), then
    tiny_clip rank 1 (6 slots) on the same array, which still holds the larger call's
    partials, then dense_small rank 3 (3 slots)."""
    fz = _fz()
    sizes = []
    for name, rank, extra in (("full_small", 0, 0.0), ("tiny_clip", 1, 0.0), ("dense_small", 3, 0.25)):
        w = synth.get(name)
        sizes.append(otable.build(w.shapes, w.dp, rank, otable.BLOCK)["shard_slots"])
        print(f"# noalloc: {name} rank {rank} ({sizes[-1]} slots)", flush=True)
        st = _pair(fz, w, rank, w.steps, extra)
        assert 0 < st["k"] < 1, name  # clipping active: the partials decide k
        if name == "full_small":
            assert st["skipped_total"] == 1
    assert sizes[0] > sizes[1] > sizes[2]


def test_noalloc_refusals():
    fz = _fz()
    w = synth.get("tiny")
    t = fz.fp8z1_build_table(w.shapes, w.dp, 0, fz.SPLIT_BLOCK)
    n = t.shard_slots
    f = lambda: torch.zeros(n * 16384, dtype=torch.float32, device="cuda")
    state = torch.zeros(8, dtype=torch.float64, device="cuda")
    grads = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in w.shapes]
    args = (fz.Hparams.make(w.hp), state, grads, f(), f(), f(), torch.zeros(n * 16384, dtype=torch.uint8, device="cuda"),
            torch.zeros(n, dtype=torch.float32, device="cuda"))
    with pytest.raises(fz.Fp8z1Error, match="not set up on a device"):
        fz.fp8z1_step_rowmajor_noalloc(t, *args)
    # a shard beyond the limit: refused from the table alone, before any buffer is used
    big = fz.fp8z1_build_table([(1, 128 * 520, 128 * 520)], 1, 0, fz.SPLIT_BLOCK)
    assert big.shard_slots > fz.NOALLOC_MAX_SLOTS
    from blockwise_fp8_zero_fold_amd import _lib
    rc = _lib.lib.fp8z1_step_rowmajor_noalloc(big.handle, _lib.C.byref(args[0]), None, None, None, None, None, None,
                                              None, None)
    assert rc == -1  # NULL grads first
    ptrs = (_lib.C.c_void_p * 1)(None)
    rc = _lib.lib.fp8z1_step_rowmajor_noalloc(big.handle, _lib.C.byref(args[0]), None, ptrs, None, None, None, None,
                                              None, None)
    assert rc == -4, rc  # FP8Z1_ESHAPE
    assert "FP8Z1_NOALLOC_MAX_SLOTS" in _lib.lib.fp8z1_last_error().decode()
    big.free()
    t.free()


def test_noalloc_step_captured_in_a_graph():
    """The callers the entry point is for: the no-alloc step captured once into a HIP
    graph (full_small: clipping, loss scaling, an inf grad that skips step 3) and
    replayed step after step with new grads copied into the captured buffers; after
    every replay the state and folded buffers equal those of an eager twin shard stepped
    by fp8z1_step_rowmajor with a workspace, bit for bit."""
    fz = _fz()
    from blockwise_fp8_zero_fold_amd.shard import Shard
    from tests import gpu_harness as gh

    w = synth.get("full_small")
    tab = otable.build(w.shapes, w.dp, 0, otable.BLOCK)
    held = gh.held_experts(tab["entries"])
    masters = gh.master_tensors(w, held)
    a, b = Shard(w.shapes, w.dp, 0), Shard(w.shapes, w.dp, 0)
    for sh in (a, b):
        sh.init(fz.Hparams.make(w.hp), masters, fz.BF16)
    n = a.n_slots
    hp = fz.Hparams.make(w.hp)
    grads = gh.grad_tensors(w, held, 1)  # the captured grad buffers

    def noalloc():
        fz.fp8z1_step_rowmajor_noalloc(b.table, hp, b.state, grads, b.master, b.m, b.v, b.fp8, b.scales)

    noalloc()  # eager step 1 (uploads this grad pointer list)
    a.update_rowmajor(hp, grads)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        noalloc()
    torch.cuda.synchronize()
    for t in range(2, w.steps + 1):
        new = gh.grad_tensors(w, held, t)
        for dst, src in zip(grads, new):
            if dst is not None:
                dst.copy_(src)
        torch.cuda.synchronize()
        g.replay()
        a.update_rowmajor(hp, grads)
        torch.cuda.synchronize()
        tag = f"graph replay for step {t}"
        sa, sb = a.read_state(), b.read_state()
        assert sa == sb, (tag, sa, sb)
        for name in ("master", "m", "v"):
            assert gh.bits_equal(gh.folded(getattr(a, name), n), gh.folded(getattr(b, name), n)), f"{tag}: {name}"
        assert gh.bits_equal(gh.folded(a.fp8, n, np.uint8), gh.folded(b.fp8, n, np.uint8)), f"{tag}: codes"
        assert gh.bits_equal(a.scales.cpu().numpy()[:n], b.scales.cpu().numpy()[:n]), f"{tag}: scales"
    assert sb["skipped_total"] == 1 and 0 < sb["k"] < 1
    del g
