"""CPU checks of the C-ABI library: it loads, exports every declared symbol, and its
host-only table builder is byte-identical to the oracle's table.  No GPU calls."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
from oracle import table as otable

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include"))) if h.endswith(".h")]

fz = pytest.importorskip("blockwise_fp8_zero_fold_amd", reason="libfp8z1.so not built")


def _declared():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8z1_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert "fp8z1_step" in names and len(names) >= 14
    for n in names:
        assert hasattr(fz.lib, n), n
    # the symbols are plain C names (no C++ mangling)
    nm = os.popen(f"nm -D --defined-only {fz.lib_path}").read()
    for n in names:
        assert re.search(rf"\bT {n}$", nm, flags=re.M), n


def _cmp(w_shapes, dp, rank, split):
    t = fz.fp8z1_build_table(w_shapes, dp, rank, split)
    o = otable.build(w_shapes, dp, rank, split)
    assert t.entries().tobytes() == o["entries"].tobytes()
    for k in ("split", "dp", "rank", "slots_per_rank", "total_blocks", "shard_first_slot", "shard_slots",
              "valid_elems", "pad_elems"):
        assert t.info[k] == o[k], k
    assert t.info["n_params"] == len(w_shapes)


@pytest.mark.parametrize("name", ["tiny", "tiny_clip", "dense_small", "moe_small", "ragged_small", "full_small"])
@pytest.mark.parametrize("split", [0, 1])
def test_table_matches_oracle_all_ranks(name, split):
    w = synth.get(name)
    for r in list(range(w.dp)) + [otable.ALL_RANKS]:
        _cmp(w.shapes, w.dp, r, split)


@pytest.mark.parametrize("name,rank", [("dense", 3), ("moe", 5), ("full", 0), ("ragged", 7), ("ragged", 15)])
@pytest.mark.parametrize("split", [0, 1])
def test_table_matches_oracle_full_size(name, rank, split):
    w = synth.get(name)
    _cmp(w.shapes, w.dp, rank, split)


def test_random_tables_match_oracle():
    rng = np.random.default_rng(21)
    for _ in range(40):
        n = int(rng.integers(1, 12))
        shapes = [(int(rng.integers(1, 4)), int(rng.integers(1, 600)), int(rng.integers(1, 600))) for _ in range(n)]
        dp = int(rng.integers(1, 9))
        for split in (0, 1):
            _cmp(shapes, dp, int(rng.integers(0, dp)), split)


def test_build_table_rejects_bad_arguments():
    good = [(1, 128, 128)]
    bad_cases = [
        (good, 0, 0, 0),        # dp < 1
        (good, 2, 2, 0),        # rank >= dp
        (good, 2, -2, 0),       # rank < -1
        (good, 2, 0, 7),        # unknown split
        ([(1, 0, 128)], 1, 0, 0),  # empty dimension
        ([(1, 1 << 23, 128)], 1, 0, 0),  # R too large for the 16-bit block row
    ]
    for shapes, dp, rank, split in bad_cases:
        with pytest.raises(fz.Fp8z1Error):
            fz.fp8z1_build_table(shapes, dp, rank, split)
    out = ctypes.c_void_p()
    assert fz.lib.fp8z1_build_table(None, 0, 1, 0, 0, ctypes.byref(out)) == -1
    assert out.value is None
    assert b"n_params" in fz.lib.fp8z1_last_error()


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        assert fz.lib.fp8z1_status_string(code)
    assert fz.lib.fp8z1_status_string(-99) == b"unknown status"


def test_argument_errors_before_any_gpu_work():
    """Calls with bad arguments fail in the host checks and never reach HIP."""
    t = fz.fp8z1_build_table([(1, 256, 256)], 1, 0)
    hp = fz.Hparams.make(synth.Hparams())
    with pytest.raises(fz.Fp8z1Error, match="NULL"):
        fz.fp8z1_fold(t, [None], fz.F32, 16, stream=0)
    with pytest.raises(fz.Fp8z1Error, match="src_dtype"):
        fz.fp8z1_fold(t, [16], 9, 16, stream=0)
    with pytest.raises(fz.Fp8z1Error, match="misaligned"):
        fz.fp8z1_fold(t, [18], fz.F32, 16, stream=0)
    with pytest.raises(fz.Fp8z1Error, match="NULL"):
        fz.fp8z1_step(t, hp, 16, 16, 16, 16, None, 16, 16, stream=0)
    with pytest.raises(fz.Fp8z1Error, match="16-byte"):
        fz.fp8z1_step(t, hp, 16, 16, 16, 16, 24, 16, 16, stream=0)
    hp_clip = fz.Hparams.make(synth.Hparams(max_grad_norm=1.0))
    with pytest.raises(fz.Fp8z1Error, match="workspace"):
        fz.fp8z1_step(t, hp_clip, 16, 16, 16, 16, 16, 16, 16, stream=0)
    with pytest.raises(fz.Fp8z1Error, match="workspace"):
        fz.fp8z1_step(t, hp_clip, 16, 16, 16, 16, 16, 16, 16, workspace=16, workspace_bytes=8, stream=0)
    hp_rule = fz.Hparams.make(synth.Hparams(scale_rule=5))
    with pytest.raises(fz.Fp8z1Error, match="scale_rule"):
        fz.fp8z1_step(t, hp_rule, 16, 16, 16, 16, 16, 16, 16, stream=0)
    hp_bad = fz.Hparams.make(synth.Hparams(beta1=1.0))
    with pytest.raises(fz.Fp8z1Error, match="betas"):
        fz.fp8z1_step(t, hp_bad, 16, 16, 16, 16, 16, 16, 16, stream=0)
    hp_nan = fz.Hparams.make(synth.Hparams(max_grad_norm=float("nan")))
    with pytest.raises(fz.Fp8z1Error, match="max_grad_norm is NaN"):
        fz.fp8z1_step(t, hp_nan, 16, 16, 16, 16, 16, 16, 16, workspace=16, stream=0)
    for bad in (dict(growth_factor=0.0), dict(backoff_factor=-0.5), dict(growth_factor=float("inf")),
                dict(backoff_factor=float("nan"))):
        hp_ls = fz.Hparams.make(synth.Hparams(loss_scaling=True, **bad))
        with pytest.raises(fz.Fp8z1Error, match="growth_factor and backoff_factor"):
            fz.fp8z1_step_rowmajor(t, hp_ls, 16, [16], 16, 16, 16, 16, 16, workspace=16, stream=0)
    with pytest.raises(fz.Fp8z1Error, match="NULL or misaligned"):
        fz.fp8z1_step_rowmajor(t, hp, 16, [None], 16, 16, 16, 16, 16, stream=0)
    with pytest.raises(fz.Fp8z1Error, match="NULL or misaligned"):
        fz.fp8z1_step_rowmajor(t, hp, 16, [18], 16, 16, 16, 16, 16, stream=0)
    with pytest.raises(fz.Fp8z1Error, match="workspace"):
        fz.fp8z1_step_rowmajor(t, hp_clip, 16, [16], 16, 16, 16, 16, 16, stream=0)
    with pytest.raises(fz.Fp8z1Error, match="NULL"):
        fz.fp8z1_fold(t, [16], fz.F32, None, stream=0)
    with pytest.raises(fz.Fp8z1Error, match="statistics-only"):
        fz.fp8z1_fold(t, [16], fz.BF16, None, slot_sumsq=16, stream=0)
    with pytest.raises(fz.Fp8z1Error, match="NULL"):
        fz.fp8z1_shard_sumsq(t, None, 16, stream=0)
    with pytest.raises(fz.Fp8z1Error, match="aligned"):
        fz.fp8z1_shard_sumsq(t, 16, 20, stream=0)
    hp_glob = fz.Hparams.make(synth.Hparams(max_grad_norm=1.0), global_sumsq=20)
    with pytest.raises(fz.Fp8z1Error, match="d_global_sumsq"):
        fz.fp8z1_step(t, hp_glob, 16, 16, 16, 16, 16, 16, 16, stream=0)
    with pytest.raises(fz.Fp8z1Error, match="dtype"):
        fz.fp8z1_unfold(t, 16, fz.BF16, None, [16], stream=0)
    with pytest.raises(fz.Fp8z1Error, match="NULL"):
        fz.fp8z1_unfold(t, 16, fz.E4M3, None, [None], stream=0)
    t.free()


def test_workspace_bytes_and_constants_match_header():
    text = "".join(open(h).read() for h in HEADERS)
    defs = dict(re.findall(r"#define (FP8Z1_[A-Z0-9_]+) \(?(-?\d+)\)?", text))
    for name, val in (("F32", fz.F32), ("BF16", fz.BF16), ("E4M3", fz.E4M3), ("SCALE_AMAX", fz.SCALE_AMAX),
                      ("SCALE_POW2", fz.SCALE_POW2), ("SPLIT_BLOCK", fz.SPLIT_BLOCK), ("SPLIT_PARAM", fz.SPLIT_PARAM),
                      ("ALL_RANKS", fz.ALL_RANKS), ("STAT_PARTS", fz.STAT_PARTS),
                      ("NOALLOC_MAX_SLOTS", fz.NOALLOC_MAX_SLOTS)):
        assert int(defs["FP8Z1_" + name]) == val, name
    for name in ("tiny", "ragged_small"):
        w = synth.get(name)
        t = fz.fp8z1_build_table(w.shapes, w.dp, 0, 0)
        assert fz.fp8z1_step_workspace_bytes(t) == 8 * fz.STAT_PARTS * t.shard_slots


def test_concurrent_table_builds_and_error_strings():
    """Threads building tables and hitting argument errors at the same time: every
    table equals the oracle's and every error message is the calling thread's own
    (the detail string is thread-local)."""
    import threading
    errors = []

    def worker(seed):
        try:
            rng = np.random.default_rng(seed)
            for i in range(60):
                n = int(rng.integers(1, 6))
                shapes = [(int(rng.integers(1, 3)), int(rng.integers(1, 500)), int(rng.integers(1, 500)))
                          for _ in range(n)]
                dp = int(rng.integers(1, 6))
                _cmp(shapes, dp, int(rng.integers(0, dp)), i % 2)
                bad, expect = ((shapes, 0, 0, 0), "dp must be") if seed % 2 else ((shapes, dp, 0, 7), "split must be")
                try:
                    fz.fp8z1_build_table(*bad)
                    errors.append((seed, "no error"))
                except fz.Fp8z1Error as e:
                    if expect not in str(e):
                        errors.append((seed, str(e)))
        except Exception as e:  # noqa: BLE001 - report any failure from the thread
            errors.append((seed, repr(e)))

    threads = [threading.Thread(target=worker, args=(s,)) for s in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:5]


def test_probe_argument_errors():
    with pytest.raises(fz.Fp8z1Error, match="parts must be"):
        fz.fp8z1_probe_update_pattern(16, 16, 16, 16, 16, 4, parts=3, stream=0)
    assert fz.lib.fp8z1_probe_copy(16, 16, 100, 1, None) == -1  # FP8Z1_EINVAL: not a multiple of 4096
    assert "multiple of 4096" in fz.lib.fp8z1_last_error().decode()
