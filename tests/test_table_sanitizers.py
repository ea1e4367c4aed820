"""The host table builder compiled for the CPU with AddressSanitizer and
UndefinedBehaviorSanitizer (g++, no GPU code), run on many shapes and compared
with the oracle's table; also fed invalid arguments."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import synth
from oracle import table as otable

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "native")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("san") / "table_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-x", "c++", os.path.join(HERE, "table_driver.c"), "-x", "none",
           os.path.join(ROOT, "blockwise_fp8_zero_fold_amd", "csrc", "table.cpp"),
           os.path.join(HERE, "table_free_stub.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail(f"sanitizer build failed:\n{r.stderr}")
    return out


def _run(driver, shapes, dp, rank, split):
    inp = f"{len(shapes)} {dp} {rank} {split}\n" + "".join(f"{e} {r} {c}\n" for e, r, c in shapes)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([driver], input=inp, capture_output=True, text=True, env=env)
    assert r.returncode == 0 and "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    return r.stdout.splitlines()


def test_sanitized_tables_match_oracle(driver):
    cases = [(synth.get(n).shapes, synth.get(n).dp) for n in ("tiny", "dense_small", "moe_small", "ragged_small")]
    rng = np.random.default_rng(31)
    for _ in range(10):
        k = int(rng.integers(1, 8))
        cases.append(([(int(rng.integers(1, 4)), int(rng.integers(1, 500)), int(rng.integers(1, 500)))
                       for _ in range(k)], int(rng.integers(1, 7))))
    for shapes, dp in cases:
        for split in (0, 1):
            for rank in list(range(dp)) + [-1]:
                lines = _run(driver, shapes, dp, rank, split)
                o = otable.build(shapes, dp, rank, split)
                info = list(map(int, lines[0].split()[1:]))
                assert info == [o["total_blocks"], o["slots_per_rank"], o["shard_first_slot"], o["shard_slots"],
                                o["valid_elems"], o["pad_elems"]]
                got = np.array([list(map(int, l.split())) for l in lines[1:]], dtype=np.int64).reshape(-1, 6)
                e = o["entries"]
                want = np.stack([e["param"], e["expert"], e["brow"], e["bcol"], e["vrows"], e["vcols"]], 1)
                assert (got == want).all()


def test_sanitized_invalid_arguments(driver):
    for shapes, dp, rank, split in [([(1, 128, 128)], 0, 0, 0), ([(1, 128, 128)], 2, 5, 0),
                                    ([(0, 128, 128)], 1, 0, 0), ([(1, 1 << 23, 8)], 1, 0, 0),
                                    ([(1, 128, 128)], 1, 0, 3)]:
        lines = _run(driver, shapes, dp, rank, split)
        assert lines[0].startswith("error -")
