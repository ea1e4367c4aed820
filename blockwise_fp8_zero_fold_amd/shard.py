"""One rank's shard: the folded device buffers (allocated with torch) and the
call sequence of the step ("面向 Blockwise FP8 量化的 ZeRO 优化器设计", section
"总结"): fold the weights into the FP32 master at init; per step fold the
reduced grads, update + requantize, unfold the FP8 codes and scales.

Buffer ownership and call order only: all arithmetic runs in libfp8z1.
"""
from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import _lib as L

BLOCK_ELEMS = 128 * 128


class Shard:
    def __init__(self, shapes: Sequence[Sequence[int]], dp: int, rank: int, split: int = L.SPLIT_BLOCK,
                 device: str = "cuda"):
        self.shapes = [tuple(int(v) for v in s) for s in shapes]
        self.table = L.fp8z1_build_table(self.shapes, dp, rank, split)
        n = self.table.shard_slots
        self.n_slots = n
        dev = torch.device(device)
        f32 = dict(dtype=torch.float32, device=dev)
        # the four float32 shard buffers back to back in one allocation: on
        # MI355X the update of the MoE expert shard ran 2 % faster so than with
        # four separate allocations, whose relative placement is left to the
        # allocator
        self._fp32 = torch.zeros(4 * n * BLOCK_ELEMS, **f32)
        self.grad, self.master, self.m, self.v = self._fp32.view(4, n * BLOCK_ELEMS).unbind(0)
        self.fp8 = torch.zeros(n * BLOCK_ELEMS, dtype=torch.uint8, device=dev)
        self.scales = torch.zeros(max(n, 1), **f32)
        self.workspace = torch.zeros(max(n * L.STAT_PARTS, 1), dtype=torch.float64, device=dev)
        self.state = torch.zeros(8, dtype=torch.float64, device=dev)  # 64 bytes

    def held_params(self):
        return L._held_params(self.table)

    def init(self, hp: L.Hparams, weights: Sequence[Optional[torch.Tensor]], dtype: int = L.F32,
             stream=None) -> None:
        """Fold the row-major weights into the FP32 master, zero m and v, reset the state."""
        L.fp8z1_fold(self.table, weights, dtype, self.master, stream=stream)
        self.m.zero_()
        self.v.zero_()
        L.fp8z1_state_init(hp, self.state, stream=stream)

    def fold_grads(self, hp: L.Hparams, grads: Sequence[Optional[torch.Tensor]], fused_stats: bool = True,
                   stream=None) -> bool:
        """Fold the reduced row-major FP32 grads; with fused_stats (and statistics on) the
        fold also writes the per-part sums of squares.  Returns whether it did."""
        stats = hp.max_grad_norm > 0 or hp.loss_scaling
        pre = bool(fused_stats and stats)
        L.fp8z1_fold(self.table, grads, L.F32, self.grad, slot_sumsq=self.workspace if pre else None,
                     stream=stream)
        return pre

    def update(self, hp: L.Hparams, presummed: bool = False, stream=None) -> None:
        L.fp8z1_step(self.table, hp, self.state, self.grad, self.master, self.m, self.v, self.fp8, self.scales,
                     workspace=self.workspace, presummed=presummed, stream=stream)

    def unfold(self, codes: Sequence[Optional[torch.Tensor]], scales: Optional[Sequence] = None,
               stream=None) -> None:
        L.fp8z1_unfold(self.table, self.fp8, L.E4M3, self.scales if scales is not None else None, codes, scales,
                       stream=stream)

    def update_rowmajor(self, hp: L.Hparams, grads: Sequence[Optional[torch.Tensor]], stream=None) -> None:
        """Update + requant reading the row-major grads directly (fold on read)."""
        L.fp8z1_step_rowmajor(self.table, hp, self.state, grads, self.master, self.m, self.v, self.fp8, self.scales,
                              workspace=self.workspace, stream=stream)

    def step(self, hp: L.Hparams, grads, codes, scales=None, fused_stats: bool = True, fold_on_read: bool = False,
             stream=None) -> None:
        """The whole per-step path: fold grads -> update + requant -> unfold (or, with
        fold_on_read, update + requant reading the row-major grads -> unfold)."""
        if fold_on_read:
            self.update_rowmajor(hp, grads, stream=stream)
        else:
            pre = self.fold_grads(hp, grads, fused_stats=fused_stats, stream=stream)
            self.update(hp, presummed=pre, stream=stream)
        self.unfold(codes, scales, stream=stream)

    def read_state(self, stream=None) -> dict:
        return L.fp8z1_state_read(self.state, stream=stream)
