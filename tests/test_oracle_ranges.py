"""CPU: the oracle run over contiguous slot ranges (what the full-size GPU check uses,
one range per worker process) gives exactly the whole-shard oracle run: the same
state after every step and the same folded master, m, v, codes and scales."""
import numpy as np
import pytest

import synth
from tests import harness
from tests import oracle_ranges as orr


@pytest.mark.parametrize("name,parts", [("full_small", 3), ("moe_small", 5), ("ragged_small", 4),
                                        ("tiny", 2), ("tiny_lossscale", 2), ("dense_small", 3)])
def test_ranges_equal_whole_shard(name, parts):
    w = synth.get(name)
    rank = w.ranks[-1]
    ref, tabs = harness.run_sharded_all_ranks(w, ranks=[rank])
    n = tabs[rank]["shard_slots"]
    rr = orr.ranges(n, parts)
    assert rr[0][0] == 0 and rr[-1][1] == n and all(a[1] == b[0] for a, b in zip(rr, rr[1:]))
    stats = w.hp.max_grad_norm > 0 or w.hp.loss_scaling
    extras = [None] * len(rr)
    if stats:
        sums = [orr.range_sumsq((name, rank, w.split, a, b, w.steps)) for a, b in rr]
        other = None
        if w.dp > 1:  # every param's whole grads minus this shard's
            whole = [orr.slab_sumsq((name, p, e, w.steps)) for p, (E, _, _) in enumerate(w.shapes) for e in range(E)]
            other = [sum(s[t] for s in whole) - sum(s[t] for s in sums) for t in range(w.steps)]
        extras = orr.extras_for(sums, other)
    res = [orr.range_run((name, rank, w.split, a, b, w.steps, extras[i], None)) for i, (a, b) in enumerate(rr)]
    last = ref[rank][w.steps - 1]
    for t in range(w.steps):
        for key, val in res[0]["states"][t].items():
            assert val == ref[rank][t]["state"][key], (name, t, key)
    for key in ("master", "m", "v", "codes", "scales"):
        for (a, b), r in zip(rr, res):
            assert r[key] == orr.digest(last[key][a:b]), (name, key, a, b)
    if name in ("full_small", "tiny_lossscale"):
        assert any(ref[rank][t]["state"]["found_inf"] for t in range(w.steps)), "the skipped step must be covered"


def test_extras_make_every_range_skip_together():
    sums = [[1.0, float("inf")], [2.0, 3.0]]
    ex = orr.extras_for(sums, other=[4.0, 5.0])
    assert ex[0][0] == 6.0 and ex[1][0] == 5.0
    assert np.isinf(ex[0][1]) and np.isinf(ex[1][1])
