"""Shard lookup table: block-wise and param-wise splits.  Test infrastructure only.

[FP8-ZeRO1] section "块粒度切分" (block-wise split): parameters are cut in
128x128 units, each quantized dimension is padded up to a multiple of 128,
and a lookup table records the real element counts and the padding so the
optimizer can walk the parameters inside a 1-D buffer.  Section
"参数粒度切分" (param-wise split): parameters are sorted by size, spread over
DP buckets by a greedy rule, and every bucket is padded up to the size of the
largest one.

Readings taken where the pages are silent (the figures are lost):
  * blocks of a param are listed in (expert, block_row, block_col) order,
    params in their given order (the order of the fold's output, section
    "参数布局变换");
  * a 2-D param has E = 1;
  * padding sits at the high end of R and of C;
  * block-wise: DP equal contiguous ranges of ceil(nb/DP) slots, the empty
    slots at the global tail;
  * param-wise: size = padded block count; LPT order (size descending, id
    ascending); each param to the least loaded bucket, lowest index on ties;
    a bucket lists its params by ascending id, then padding slots up to the
    largest bucket; bucket r is rank r.

One table entry per slot, 16 bytes: int32 param (-1 = padding slot),
int32 expert, uint16 block_row, uint16 block_col, uint8 valid_rows,
uint8 valid_cols, uint16 reserved (0).
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

BLOCK = 0
PARAM = 1
ALL_RANKS = -1
B = 128

ENTRY_DTYPE = np.dtype([
    ("param", "<i4"), ("expert", "<i4"), ("brow", "<u2"), ("bcol", "<u2"),
    ("vrows", "u1"), ("vcols", "u1"), ("reserved", "<u2")])
assert ENTRY_DTYPE.itemsize == 16


def grid(shape: Tuple[int, int, int]) -> Tuple[int, int, int]:
    """(E, Rb, Cb): experts and block rows/cols after padding each of R, C to a multiple of 128."""
    e, r, c = shape
    return e, -(-r // B), -(-c // B)


def param_block_list(pid: int, shape: Tuple[int, int, int]) -> List[Tuple[int, int, int, int, int, int]]:
    """All blocks of one param in (expert, block_row, block_col) order, with their valid extents."""
    e_n, r, c = shape
    _, rb, cb = grid(shape)
    out = []
    for e in range(e_n):
        for br in range(rb):
            for bc in range(cb):
                out.append((pid, e, br, bc, min(B, r - B * br), min(B, c - B * bc)))
    return out


def _pad_entry():
    return (-1, 0, 0, 0, 0, 0)


def lpt_assign(sizes: Sequence[int], dp: int) -> List[int]:
    """Greedy param-wise split: bucket index for every param."""
    order = sorted(range(len(sizes)), key=lambda i: (-sizes[i], i))
    loads = [0] * dp
    owner = [0] * len(sizes)
    for i in order:
        b = min(range(dp), key=lambda j: (loads[j], j))
        owner[i] = b
        loads[b] += sizes[i]
    return owner


def global_slots(shapes: Sequence[Tuple[int, int, int]], dp: int, split: int):
    """The whole flat slot list (all ranks) and the number of slots per rank."""
    if split == BLOCK:
        blocks = []
        for pid, s in enumerate(shapes):
            blocks += param_block_list(pid, s)
        nb = len(blocks)
        spr = -(-nb // dp) if nb else 0
        slots = blocks + [_pad_entry()] * (dp * spr - nb)
        return slots, spr
    if split == PARAM:
        sizes = [int(np.prod(grid(s))) for s in shapes]
        owner = lpt_assign(sizes, dp)
        loads = [0] * dp
        for i, b in enumerate(owner):
            loads[b] += sizes[i]
        spr = max(loads) if loads else 0
        slots = []
        for b in range(dp):
            mine = []
            for pid in range(len(shapes)):
                if owner[pid] == b:
                    mine += param_block_list(pid, shapes[pid])
            slots += mine + [_pad_entry()] * (spr - len(mine))
        return slots, spr
    raise ValueError("split must be BLOCK or PARAM")


def build(shapes: Sequence[Tuple[int, int, int]], dp: int, rank: int, split: int = BLOCK) -> dict:
    """Table of one rank's shard (rank = ALL_RANKS: the whole flat buffer)."""
    if dp < 1 or not (rank == ALL_RANKS or 0 <= rank < dp):
        raise ValueError("bad dp/rank")
    slots, spr = global_slots(shapes, dp, split)
    if rank == ALL_RANKS:
        first, n = 0, dp * spr
    else:
        first, n = rank * spr, spr
    ent = np.zeros(n, dtype=ENTRY_DTYPE)
    for k in range(n):
        p, e, br, bc, vr, vc = slots[first + k]
        ent[k] = (p, e, br, bc, vr, vc, 0)
    valid = int(np.sum(ent["vrows"].astype(np.int64) * ent["vcols"].astype(np.int64)))
    return {
        "entries": ent, "split": split, "dp": dp, "rank": rank, "shapes": [tuple(s) for s in shapes],
        "slots_per_rank": spr, "total_blocks": sum(int(np.prod(grid(s))) for s in shapes),
        "shard_first_slot": first, "shard_slots": n, "valid_elems": valid,
        "pad_elems": n * B * B - valid,
    }


def even_1d_split_cuts_blocks(shapes: Sequence[Tuple[int, int, int]], dp: int) -> int:
    """Number of 128x128 blocks that the plain flatten-and-split-evenly ZeRO layout
    ([FP8-ZeRO1] sections "ZeRO-1 优化器" and the first challenge) spreads over
    more than one rank.  Row-major flattening, the buffer cut into DP equal
    ranges of ceil(N/DP) elements."""
    offs = []
    base = 0
    for s in shapes:
        offs.append(base)
        base += s[0] * s[1] * s[2]
    per = -(-base // dp)
    cut = 0
    for pid, (e_n, r, c) in enumerate(shapes):
        for e, br, bc in ((e, br, bc) for e in range(e_n) for br in range(-(-r // B)) for bc in range(-(-c // B))):
            owners = set()
            for i in range(B * br, min(r, B * br + B)):
                lo = offs[pid] + (e * r + i) * c + B * bc
                hi = lo + min(B, c - B * bc) - 1
                owners.add(lo // per)
                owners.add(hi // per)
            if len(owners) > 1:
                cut += 1
    return cut
