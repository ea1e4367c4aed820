"""GPU parity on every element of full-size shards, in the launch configurations
bench.py times (update reading the row-major grads, and fold with fused statistics
then update; then unfold), both routes fed the same grads.

The oracle runs in 16 worker processes, each over one contiguous slot range of the
shard (blocks are independent once the global statistics are known; each range gets
the rest of the shard's sum of squares, plus the other ranks' sum, as its extra
term; the other ranks' sum is the sum over every param's whole grads minus the
shard's, and the GPU step gets it as its extra term too).  The workers return the
state after every step and digests of their final folded master, m, v, codes and
scales; the test hashes the same slot ranges of the GPU's folded buffers, and of
the GPU's unfolded row-major codes and scales brought back into slot order by the
oracle's own fold, and requires every digest to match."""
import multiprocessing as mp
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import synth
from oracle import layout, optim, table as otable
from tests import harness, oracle_ranges as orr

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BLOCK = 128 * 128
WORKERS = 16  # the host share of one GPU


def _fz():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import blockwise_fp8_zero_fold_amd as fz
    return fz


def _upload(w, held, make, dtype=torch.float32):
    """Row-major device tensors of the held params, the held experts drawn on host threads."""
    need = [(p, e) for p, es in held.items() for e in es]
    out = [torch.zeros(s, dtype=dtype, device="cuda") if p in held else None for p, s in enumerate(w.shapes)]
    with ThreadPoolExecutor(WORKERS) as ex:
        for (p, e), slab in zip(need, ex.map(lambda pe: make(*pe), need)):
            if dtype == torch.bfloat16:
                out[p][e].copy_(torch.from_numpy(slab.view(np.int16)).view(torch.bfloat16))
            else:
                out[p][e].copy_(torch.from_numpy(slab))
    return out


def _range_digests(host: np.ndarray, rr, unit: int):
    with ThreadPoolExecutor(WORKERS) as ex:
        return list(ex.map(lambda ab: orr.digest(host[ab[0] * unit:ab[1] * unit]), rr))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,steps,split", [("moe", 5, None), ("full", 5, None), ("ragged", 3, None),
                                              ("ragged", 3, "param"), ("dense", 10, None)])
def test_every_element_full_size(name, steps, split):
    fz = _fz()
    from blockwise_fp8_zero_fold_amd.shard import Shard
    from tests import gpu_harness as gh

    w = synth.get(name)
    if split:
        w = w.with_(split=split)
    rank = w.ranks[0]
    tab = otable.build(w.shapes, w.dp, rank, otable.PARAM if w.split == "param" else otable.BLOCK)
    ent = tab["entries"]
    nslots = len(ent)
    rr = orr.ranges(nslots, WORKERS)
    stats = w.hp.max_grad_norm > 0 or w.hp.loss_scaling
    print(f"[{name}] rank {rank}: {nslots} slots in {len(rr)} oracle ranges, {steps} steps", flush=True)

    ctx = mp.get_context("spawn")  # fresh interpreters: the workers never touch the GPU
    with ctx.Pool(len(rr)) as pool:
        other = None
        if stats:
            sums = pool.map_async(orr.range_sumsq, [(name, rank, w.split, a, b, steps) for a, b in rr])
            if w.dp > 1:
                whole = pool.map(orr.slab_sumsq, [(name, p, e, steps) for p, (E, _, _) in enumerate(w.shapes)
                                                  for e in range(E)])
                mine = sums.get(timeout=600)
                other = [sum(s[t] for s in whole) - sum(s[t] for s in mine) for t in range(steps)]

        split = fz.SPLIT_PARAM if w.split == "param" else fz.SPLIT_BLOCK
        routes = {True: Shard(w.shapes, w.dp, rank, split), False: Shard(w.shapes, w.dp, rank, split)}
        held = gh.held_experts(ent)
        if w.master_dtype == "bf16":
            weights = _upload(w, held, lambda p, e: synth.master_slab_bf16(w, p, e), torch.bfloat16)
        else:
            weights = _upload(w, held, lambda p, e: synth.master_slab(w, p, e))
        for sh in routes.values():
            assert sh.table.entries().tobytes() == ent.tobytes()
            sh.init(fz.Hparams.make(w.hp), weights, fz.BF16 if w.master_dtype == "bf16" else fz.F32)
        del weights
        dst = {r: gh.code_tensors(w, held) for r in routes}
        gpu_states = {r: [] for r in routes}
        for t in range(1, steps + 1):
            hp = fz.Hparams.make(w.hp, extra_sumsq=other[t - 1]) if other else fz.Hparams.make(w.hp)
            grads = _upload(w, held, lambda p, e: synth.grad_slab(w, p, e, t))
            for r, sh in routes.items():
                sh.step(hp, grads, dst[r][0], dst[r][1], fused_stats=True, fold_on_read=r)
                gpu_states[r].append(sh.read_state())
            del grads
            print(f"[{name}] GPU step {t} done", flush=True)

        ks = None
        if stats:
            mine = sums.get(timeout=600)
            extras = orr.extras_for(mine, other)
            # two-stage clip check: the sums within 1e-12, and where the GPU's k differs
            # from the oracle's (another summation order) the oracle runs with the GPU's k
            tot = [sum(s[t] for s in mine) + (other[t] if other else 0.0) for t in range(steps)]
            st = optim.init_state(w.hp)
            ks = []
            for t in range(steps):
                want_st = optim.finalize(st, w.hp, tot[t], 0.0)
                assert gpu_states[True][t]["k"] == gpu_states[False][t]["k"], (name, "routes' k differ", t + 1)
                k = harness.clip_stage1(w.hp, st, gpu_states[True][t], want_st, f"{name} step {t + 1}")
                ks.append(k)
                st = want_st if k is None else dict(want_st, k=k)
            if all(k is None for k in ks):
                ks = None
        else:
            extras = [None] * len(rr)
        run = pool.map_async(orr.range_run, [(name, rank, w.split, a, b, steps, extras[i], ks)
                                             for i, (a, b) in enumerate(rr)])

        # the GPU's results, hashed by the same slot ranges, while the oracle runs
        got = {}
        for r, sh in routes.items():
            d = {}
            for key in ("master", "m", "v"):
                host = getattr(sh, key)[: nslots * BLOCK].cpu().numpy()
                d[key] = _range_digests(host, rr, BLOCK)
                del host
            d["codes"] = _range_digests(sh.fp8[: nslots * BLOCK].cpu().numpy(), rr, BLOCK)
            d["scales"] = _range_digests(sh.scales[:nslots].cpu().numpy(), rr, 1)
            # unfolded codes and scales, brought back into slot order by the oracle's fold
            codes = {p: dst[r][0][p].cpu().numpy() for p in held}
            scl = {p: dst[r][1][p].cpu().numpy() for p in held}
            un_c, un_s = [], []
            for a, b in rr:
                sub = dict(tab)
                sub["entries"] = ent[a:b]
                un_c.append(orr.digest(layout.fold_shard(sub, codes, dtype=np.uint8)))
                e_ = ent[a:b]
                s = np.ones(b - a, np.float32)  # the oracle's scale of a padding slot
                for p in held:
                    sel = e_["param"] == p
                    s[sel] = scl[p][e_["expert"][sel], e_["brow"][sel], e_["bcol"][sel]]
                un_s.append(orr.digest(s))
            d["unfolded codes"], d["unfolded scales"] = un_c, un_s
            del codes, scl
            got[r] = d
        print(f"[{name}] GPU results hashed", flush=True)
        want = run.get(timeout=900)
    print(f"[{name}] oracle ranges done", flush=True)

    for i, res in enumerate(want):
        for t in range(steps):
            assert res["states"][t] == want[0]["states"][t], (name, "ranges disagree", i, t)
    for r in routes:
        tag = f"{name} fold_on_read={r}"
        for t in range(steps):
            for key, val in want[0]["states"][t].items():
                assert gpu_states[r][t][key] == val, (tag, "step", t + 1, key, gpu_states[r][t][key], val)
        for key, want_key in (("master", "master"), ("m", "m"), ("v", "v"), ("codes", "codes"),
                              ("scales", "scales"), ("unfolded codes", "codes"), ("unfolded scales", "scales")):
            bad = [rr[i] for i, res in enumerate(want) if got[r][key][i] != res[want_key]]
            assert not bad, f"{tag}: {key} differ in slot ranges {bad}"
    if name == "full":
        assert any(s["found_inf"] for s in want[0]["states"]), "the skipped step must be covered"
