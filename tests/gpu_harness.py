"""GPU-side helpers for the parity tests: upload seeded row-major inputs, drive a
Shard through the library, read folded buffers back.  Expected values come from
``oracle`` only (see tests/harness.py)."""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np
import torch

import synth
from oracle import layout, table as otable

BLOCK = 128 * 128


def held_experts(entries: np.ndarray) -> Dict[int, List[int]]:
    out: Dict[int, set] = {}
    for p, e in zip(entries["param"], entries["expert"]):
        if p >= 0:
            out.setdefault(int(p), set()).add(int(e))
    return {p: sorted(s) for p, s in out.items()}


def device_params(w, held: Dict[int, List[int]], make_slab, dtype=torch.float32, fill=0.0):
    """Row-major [E,R,C] device tensors for the held params; only held experts are filled
    (from ``make_slab(pid, e)``), the rest keep ``fill``.  Unheld params are None."""
    out: List[Optional[torch.Tensor]] = []
    for pid, (E, R, C) in enumerate(w.shapes):
        if pid not in held:
            out.append(None)
            continue
        t = torch.full((E, R, C), fill, dtype=dtype, device="cuda")
        for e in held[pid]:
            slab = make_slab(pid, e)
            if dtype == torch.bfloat16:
                t[e].copy_(torch.from_numpy(slab.view(np.int16)).view(torch.bfloat16), non_blocking=False)
            else:
                t[e].copy_(torch.from_numpy(slab), non_blocking=False)
        out.append(t)
    return out


def master_tensors(w, held):
    if w.master_dtype == "bf16":
        return device_params(w, held, lambda p, e: synth.master_slab_bf16(w, p, e), torch.bfloat16)
    return device_params(w, held, lambda p, e: synth.master_slab(w, p, e))


def grad_tensors(w, held, t):
    return device_params(w, held, lambda p, e: synth.grad_slab(w, p, e, t))


def code_tensors(w, held, sentinel=0xA5):
    codes = [torch.full(s, sentinel, dtype=torch.uint8, device="cuda") if p in held else None
             for p, s in enumerate(w.shapes)]
    scales = [torch.full(otable.grid(s), float("nan"), dtype=torch.float32, device="cuda") if p in held else None
              for p, s in enumerate(w.shapes)]
    return codes, scales


def folded(x: torch.Tensor, n: int, dtype=np.float32) -> np.ndarray:
    return x.cpu().numpy().view(dtype)[: n * BLOCK].reshape(n, 128, 128)


def bits_equal(a: np.ndarray, b: np.ndarray) -> bool:
    return np.ascontiguousarray(a).tobytes() == np.ascontiguousarray(b).tobytes()


def first_diff(a: np.ndarray, b: np.ndarray):
    a = np.ascontiguousarray(a).view(np.uint8).ravel()
    b = np.ascontiguousarray(b).view(np.uint8).ravel()
    d = np.nonzero(a != b)[0]
    return None if len(d) == 0 else (int(d[0]), len(d))
