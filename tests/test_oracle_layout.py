"""Pins of the oracle's fold/unfold: the printed torch formula, round trips, index closed form."""
import numpy as np
import pytest
import torch

import synth
from oracle import layout, table


def _printed_fold(w: torch.Tensor) -> torch.Tensor:
    # the view/permute/contiguous/view sequence printed in section "参数布局变换", run in torch
    return (w.view(w.shape[0], w.shape[1] // 128, 128, w.shape[2] // 128, 128)
            .permute(0, 1, 3, 2, 4).contiguous().view(-1, 128, 128))


def _printed_unfold(wb: torch.Tensor, e, r, c) -> torch.Tensor:
    return (wb.view(e, r // 128, c // 128, 128, 128).permute(0, 1, 3, 2, 4).contiguous().view(e, r, c))


@pytest.mark.parametrize("shape", [(1, 128, 128), (1, 256, 384), (3, 384, 256), (2, 128, 640)])
def test_fold_equals_printed_formula(shape):
    x = np.random.default_rng(0).standard_normal(shape).astype(np.float32)
    ours = layout.fold_param(x)
    theirs = _printed_fold(torch.from_numpy(x)).numpy()
    assert ours.tobytes() == theirs.tobytes()
    back = layout.unfold_param(ours, shape)
    assert back.tobytes() == _printed_unfold(torch.from_numpy(ours), *shape).numpy().tobytes()


@pytest.mark.parametrize("shape", [(1, 200, 300), (2, 129, 1), (1, 1, 257), (3, 64, 130)])
def test_round_trip_bit_exact(shape):
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, size=shape, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)  # includes NaN payloads, -0, subnormals
    f = layout.fold_param(x)
    assert layout.unfold_param(f, shape).view(np.uint32).tobytes() == bits.tobytes()
    # padding is +0 (bit pattern 0)
    mask = np.zeros(f.shape, bool)
    _, rb, cb = table.grid(shape)
    k = 0
    for e in range(shape[0]):
        for br in range(rb):
            for bc in range(cb):
                mask[k, :min(128, shape[1] - 128 * br), :min(128, shape[2] - 128 * bc)] = True
                k += 1
    assert (f.view(np.uint32)[~mask] == 0).all()


def test_bf16_widen_round_trip():
    w = synth.get("full_small")
    bits = synth.master_slab_bf16(w, 0, 1)
    wide = layout.widen_bf16(bits)
    # exact: a bfloat16 value is representable in float32, and torch agrees
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert wide.tobytes() == ref.tobytes()
    x = wide[None]
    assert layout.unfold_param(layout.fold_param(x), x.shape).tobytes() == x.tobytes()


@pytest.mark.parametrize("shape", [(2, 300, 260), (1, 128, 256)])
def test_index_tensor_closed_form(shape):
    E, R, C = shape
    idx = np.arange(E * R * C, dtype=np.int64).reshape(shape)
    f = layout.fold_param(idx)
    _, rb, cb = table.grid(shape)
    k = np.arange(f.shape[0])[:, None, None]
    i = np.arange(128)[None, :, None]
    j = np.arange(128)[None, None, :]
    e, rem = k // (rb * cb), k % (rb * cb)
    br, bc = rem // cb, rem % cb
    row, col = 128 * br + i, 128 * bc + j
    want = np.where((row < R) & (col < C), (e * R + row) * C + col, 0)
    assert (f == want).all()


@pytest.mark.parametrize("name", ["tiny", "ragged_small", "moe_small"])
@pytest.mark.parametrize("split", [table.BLOCK, table.PARAM])
def test_shard_fold_unfold_all_ranks(name, split):
    w = synth.get(name)
    rng = np.random.default_rng(2)
    src = {p: rng.standard_normal(s).astype(np.float32) for p, s in enumerate(w.shapes)}
    dst = {p: np.full(s, np.nan, np.float32) for p, s in enumerate(w.shapes)}
    for r in range(w.dp):
        tab = table.build(w.shapes, w.dp, r, split)
        f = layout.fold_shard(tab, src)
        mask = layout.valid_mask(tab)
        assert (f[~mask] == 0).all()
        layout.unfold_shard(tab, f, dst)
    for p in src:
        assert dst[p].tobytes() == src[p].tobytes()
    if split == table.BLOCK:
        # block-wise: the concatenated shards are the folded params laid end to end
        whole = np.concatenate([layout.fold_param(src[p]) for p in range(len(w.shapes))])
        cat = np.concatenate([layout.fold_shard(table.build(w.shapes, w.dp, r), src) for r in range(w.dp)])
        assert cat[:len(whole)].tobytes() == whole.tobytes()
        assert (cat[len(whole):] == 0).all()
