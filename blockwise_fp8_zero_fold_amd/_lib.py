"""ctypes binding of libfp8z1.so: argument marshalling only."""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import numpy as np

# torch ships its own HIP runtime under the same soname as ROCm's.  Importing
# torch first makes libfp8z1 bind to that one runtime, so the streams and
# device pointers torch hands over belong to the runtime the library calls;
# loading the library first would map a second runtime into the process.
import torch  # noqa: F401,E402

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libfp8z1.so")

F32, BF16, E4M3 = 0, 1, 2
SCALE_AMAX, SCALE_POW2 = 0, 1
SPLIT_BLOCK, SPLIT_PARAM = 0, 1
STAT_PARTS = 4  # float64 partial sums of squares per slot
NOALLOC_MAX_SLOTS = 262144  # largest table fp8z1_step_rowmajor_noalloc takes
ALL_RANKS = -1

BLOCK_ENTRY_DTYPE = np.dtype([
    ("param", "<i4"), ("expert", "<i4"), ("brow", "<u2"), ("bcol", "<u2"),
    ("vrows", "u1"), ("vcols", "u1"), ("reserved", "<u2")])


class Fp8z1Error(RuntimeError):
    pass


if not os.path.exists(lib_path):
    raise ImportError(f"{lib_path} is not built: run `python blockwise_fp8_zero_fold_amd/build.py`")
lib = C.CDLL(lib_path)


class Shape(C.Structure):
    _fields_ = [("E", C.c_int64), ("R", C.c_int64), ("C", C.c_int64)]


class Block(C.Structure):
    _fields_ = [("param", C.c_int32), ("expert", C.c_int32), ("brow", C.c_uint16), ("bcol", C.c_uint16),
                ("vrows", C.c_uint8), ("vcols", C.c_uint8), ("reserved", C.c_uint16)]


class TableInfo(C.Structure):
    _fields_ = [("split", C.c_int32), ("dp", C.c_int32), ("rank", C.c_int32), ("n_params", C.c_int32),
                ("total_blocks", C.c_int64), ("slots_per_rank", C.c_int64), ("shard_first_slot", C.c_int64),
                ("shard_slots", C.c_int64), ("valid_elems", C.c_int64), ("pad_elems", C.c_int64)]


class Hparams(C.Structure):
    _fields_ = [("lr", C.c_float), ("beta1", C.c_float), ("beta2", C.c_float), ("eps", C.c_float),
                ("weight_decay", C.c_float), ("max_grad_norm", C.c_float), ("loss_scaling", C.c_int32),
                ("init_scale", C.c_float), ("growth_factor", C.c_float), ("backoff_factor", C.c_float),
                ("growth_interval", C.c_int32), ("extra_found_inf", C.c_int32), ("scale_rule", C.c_int32),
                ("extra_sumsq", C.c_double), ("d_global_sumsq", C.c_void_p)]

    @classmethod
    def make(cls, hp, extra_sumsq: float = 0.0, extra_found_inf: bool = False, global_sumsq=None) -> "Hparams":
        """From any object with the same attribute names (e.g. synth.Hparams).  global_sumsq:
        None, or a device float64 tensor (or address) holding the all-ranks sum of squares."""
        if global_sumsq is not None and not isinstance(global_sumsq, int):
            _need(global_sumsq, 8, "global_sumsq", torch.float64)
        out = cls(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.max_grad_norm, int(bool(hp.loss_scaling)),
                  hp.init_scale, hp.growth_factor, hp.backoff_factor, int(hp.growth_interval),
                  int(bool(extra_found_inf)), int(getattr(hp, "scale_rule", 0)), float(extra_sumsq),
                  _ptr(global_sumsq))
        out._keep = global_sumsq  # the tensor must outlive the calls that use these settings
        return out


class State(C.Structure):
    _fields_ = [("step", C.c_int64), ("beta1_pow", C.c_double), ("beta2_pow", C.c_double),
                ("global_sumsq", C.c_double), ("loss_scale", C.c_float), ("k", C.c_float),
                ("step_size", C.c_float), ("bc2_sqrt", C.c_float), ("decay", C.c_float),
                ("good_steps", C.c_int32), ("found_inf", C.c_int32), ("skipped_total", C.c_int32)]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


assert C.sizeof(Block) == 16 and C.sizeof(State) == 64 and C.sizeof(Hparams) == 72

_vp = C.c_void_p
_sig = {
    "fp8z1_status_string": (C.c_char_p, [C.c_int]),
    "fp8z1_last_error": (C.c_char_p, []),
    "fp8z1_build_table": (C.c_int, [C.POINTER(Shape), C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.POINTER(_vp)]),
    "fp8z1_table_info_get": (C.c_int, [_vp, C.POINTER(TableInfo)]),
    "fp8z1_table_entries": (C.c_int, [_vp, C.POINTER(C.POINTER(Block))]),
    "fp8z1_table_free": (None, [_vp]),
    "fp8z1_fold": (C.c_int, [_vp, C.POINTER(_vp), C.c_int32, _vp, _vp, _vp]),
    "fp8z1_state_init": (C.c_int, [C.POINTER(Hparams), _vp, _vp]),
    "fp8z1_step_workspace_bytes": (C.c_int, [_vp, C.POINTER(C.c_size_t)]),
    "fp8z1_shard_sumsq": (C.c_int, [_vp, _vp, _vp, _vp]),
    "fp8z1_step": (C.c_int, [_vp, C.POINTER(Hparams), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, C.c_size_t, C.c_int32,
                             _vp]),
    "fp8z1_step_rowmajor": (C.c_int, [_vp, C.POINTER(Hparams), _vp, C.POINTER(_vp), _vp, _vp, _vp, _vp, _vp, _vp,
                                      C.c_size_t, _vp]),
    "fp8z1_step_rowmajor_noalloc": (C.c_int, [_vp, C.POINTER(Hparams), _vp, C.POINTER(_vp), _vp, _vp, _vp, _vp,
                                              _vp, _vp]),
    "fp8z1_unfold": (C.c_int, [_vp, _vp, C.c_int32, _vp, C.POINTER(_vp), C.POINTER(_vp), _vp]),
    "fp8z1_state_read": (C.c_int, [_vp, C.POINTER(State), _vp]),
    "fp8z1_state_write": (C.c_int, [_vp, C.POINTER(State), _vp]),
    "fp8z1_encode_e4m3": (C.c_int, [_vp, _vp, C.c_int64, _vp]),
    "fp8z1_dequantize": (C.c_int, [_vp, _vp, C.c_int64, C.c_int64, C.c_int64, C.c_int32, _vp, _vp]),
    "fp8z1_probe_copy": (C.c_int, [_vp, _vp, C.c_int64, C.c_int64, _vp]),
    "fp8z1_probe_update_pattern": (C.c_int, [_vp, _vp, _vp, _vp, _vp, C.c_int64, C.c_int32, _vp]),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def _check(rc: int, what: str) -> None:
    if rc != 0:
        msg = lib.fp8z1_last_error().decode(errors="replace")
        raise Fp8z1Error(f"{what}: {lib.fp8z1_status_string(rc).decode()} ({rc}): {msg}")


def _ptr(x) -> Optional[int]:
    """Device pointer of a torch tensor (or an int address, or None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr_list(xs: Sequence) -> C.Array:
    arr = (_vp * len(xs))()
    for i, x in enumerate(xs):
        arr[i] = _ptr(x)
    return arr


class Table:
    """Owns one fp8z1_table handle."""

    def __init__(self, handle: int, shapes=None):
        self.handle = C.c_void_p(handle)
        self.shapes = [tuple(int(v) for v in s) for s in shapes] if shapes is not None else None
        info = TableInfo()
        _check(lib.fp8z1_table_info_get(self.handle, C.byref(info)), "fp8z1_table_info_get")
        self.info = {f: getattr(info, f) for f, _ in TableInfo._fields_}

    @property
    def shard_slots(self) -> int:
        return self.info["shard_slots"]

    @property
    def n_params(self) -> int:
        return self.info["n_params"]

    def entries(self) -> np.ndarray:
        """Copy of the shard's 16-byte entries as a numpy structured array."""
        p = C.POINTER(Block)()
        _check(lib.fp8z1_table_entries(self.handle, C.byref(p)), "fp8z1_table_entries")
        n = self.shard_slots
        if n == 0:
            return np.zeros(0, BLOCK_ENTRY_DTYPE)
        raw = C.string_at(p, 16 * n)
        return np.frombuffer(raw, dtype=BLOCK_ENTRY_DTYPE).copy()

    def free(self) -> None:
        if self.handle:
            lib.fp8z1_table_free(self.handle)
            self.handle = C.c_void_p(None)

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def fp8z1_build_table(shapes: Sequence[Sequence[int]], dp: int, rank: int, split: int = SPLIT_BLOCK) -> Table:
    arr = (Shape * len(shapes))(*[Shape(int(e), int(r), int(c)) for e, r, c in shapes])
    out = C.c_void_p()
    _check(lib.fp8z1_build_table(arr, len(shapes), dp, rank, split, C.byref(out)), "fp8z1_build_table")
    return Table(out.value, shapes)


# ------------------------------------------------------------------ size checks
# The C library cannot see buffer sizes; when torch tensors are passed, check
# them here so that no kernel is launched on a buffer smaller than it assumes.

def _is_tensor(x) -> bool:
    return hasattr(x, "data_ptr") and hasattr(x, "numel")


def _need(x, nbytes: int, what: str, dtype=None) -> None:
    if not _is_tensor(x):
        return
    if not x.is_cuda or not x.is_contiguous():
        raise Fp8z1Error(f"{what}: must be a contiguous device tensor")
    if dtype is not None and x.dtype != dtype:
        raise Fp8z1Error(f"{what}: dtype {x.dtype}, expected {dtype}")
    if x.numel() * x.element_size() < nbytes:
        raise Fp8z1Error(f"{what}: {x.numel() * x.element_size()} bytes, needs {nbytes}")


def _held_params(table: Table):
    held = getattr(table, "_held", None)
    if held is None:
        u = np.unique(table.entries()["param"])
        held = table._held = [int(p) for p in u if p >= 0]
    return held


def _torch_dtype(code: int):
    import torch
    return {F32: torch.float32, BF16: torch.bfloat16, E4M3: torch.uint8}[code]


def _check_param_list(table: Table, xs: Sequence, dtype: int, what: str, scales: bool = False) -> None:
    if table.shapes is None or not any(_is_tensor(x) for x in xs if x is not None):
        return
    if len(xs) != table.n_params:
        raise Fp8z1Error(f"{what}: {len(xs)} entries for {table.n_params} params")
    import torch
    el = 4 if scales else {F32: 4, BF16: 2, E4M3: 1}[dtype]
    for p in _held_params(table):
        e, r, c = table.shapes[p]
        n = e * (-(-r // 128)) * (-(-c // 128)) if scales else e * r * c
        if xs[p] is None:
            raise Fp8z1Error(f"{what}: param {p} is held by the shard but its pointer is None")
        _need(xs[p], n * el, f"{what}[{p}]", torch.float32 if scales else _torch_dtype(dtype))


def fp8z1_fold(table: Table, srcs: Sequence, src_dtype: int, dst, slot_sumsq=None, stream=None) -> None:
    """dst None with slot_sumsq given: the statistics pass alone (row-major FP32 grads)."""
    n = table.shard_slots
    if dst is not None:
        _need(dst, n * 16384 * 4, "fold dst")
    if slot_sumsq is not None:
        _need(slot_sumsq, n * STAT_PARTS * 8, "fold slot_sumsq")
    _check_param_list(table, srcs, src_dtype, "fold src")
    _check(lib.fp8z1_fold(table.handle, _ptr_list(srcs), src_dtype, _ptr(dst), _ptr(slot_sumsq), _stream(stream)),
           "fp8z1_fold")


def fp8z1_state_init(hp: Hparams, d_state, stream=None) -> None:
    _need(d_state, 64, "state")
    _check(lib.fp8z1_state_init(C.byref(hp), _ptr(d_state), _stream(stream)), "fp8z1_state_init")


def fp8z1_step_workspace_bytes(table: Table) -> int:
    n = C.c_size_t()
    _check(lib.fp8z1_step_workspace_bytes(table.handle, C.byref(n)), "fp8z1_step_workspace_bytes")
    return n.value


def fp8z1_shard_sumsq(table: Table, partials, out, stream=None) -> None:
    """Sum the shard's partial sums of squares (as fp8z1_fold wrote them) into out[0] (float64)."""
    _need(partials, table.shard_slots * STAT_PARTS * 8, "shard_sumsq partials", torch.float64)
    _need(out, 8, "shard_sumsq out", torch.float64)
    _check(lib.fp8z1_shard_sumsq(table.handle, _ptr(partials), _ptr(out), _stream(stream)), "fp8z1_shard_sumsq")


def fp8z1_step(table: Table, hp: Hparams, d_state, grad, master, m, v, fp8, scales, workspace=None,
               workspace_bytes: int = 0, presummed: bool = False, stream=None) -> None:
    if workspace is not None and not workspace_bytes and _is_tensor(workspace):
        workspace_bytes = workspace.numel() * workspace.element_size()
    n = table.shard_slots
    for name, x in (("grad", grad), ("master", master), ("m", m), ("v", v)):
        _need(x, n * 16384 * 4, f"step {name}")
    _need(fp8, n * 16384, "step fp8")
    _need(scales, n * 4, "step scales")
    _need(d_state, 64, "step state")
    if workspace is not None:
        _need(workspace, n * STAT_PARTS * 8, "step workspace")
    _check(lib.fp8z1_step(table.handle, C.byref(hp), _ptr(d_state), _ptr(grad), _ptr(master), _ptr(m), _ptr(v),
                          _ptr(fp8), _ptr(scales), _ptr(workspace), workspace_bytes, int(bool(presummed)),
                          _stream(stream)), "fp8z1_step")


def fp8z1_step_rowmajor(table: Table, hp: Hparams, d_state, grads: Sequence, master, m, v, fp8, scales,
                        workspace=None, workspace_bytes: int = 0, stream=None) -> None:
    if workspace is not None and not workspace_bytes and _is_tensor(workspace):
        workspace_bytes = workspace.numel() * workspace.element_size()
    n = table.shard_slots
    for name, x in (("master", master), ("m", m), ("v", v)):
        _need(x, n * 16384 * 4, f"step_rowmajor {name}")
    _need(fp8, n * 16384, "step_rowmajor fp8")
    _need(scales, n * 4, "step_rowmajor scales")
    _need(d_state, 64, "step_rowmajor state")
    if workspace is not None:
        _need(workspace, n * STAT_PARTS * 8, "step_rowmajor workspace")
    _check_param_list(table, grads, F32, "step_rowmajor grads")
    _check(lib.fp8z1_step_rowmajor(table.handle, C.byref(hp), _ptr(d_state), _ptr_list(grads), _ptr(master), _ptr(m),
                                   _ptr(v), _ptr(fp8), _ptr(scales), _ptr(workspace), workspace_bytes,
                                   _stream(stream)), "fp8z1_step_rowmajor")


def fp8z1_step_rowmajor_noalloc(table: Table, hp: Hparams, d_state, grads: Sequence, master, m, v, fp8, scales,
                                stream=None) -> None:
    """fp8z1_step_rowmajor without a workspace: the library keeps the statistics partials
    in its own device array, so the call allocates nothing."""
    n = table.shard_slots
    for name, x in (("master", master), ("m", m), ("v", v)):
        _need(x, n * 16384 * 4, f"step_rowmajor_noalloc {name}")
    _need(fp8, n * 16384, "step_rowmajor_noalloc fp8")
    _need(scales, n * 4, "step_rowmajor_noalloc scales")
    _need(d_state, 64, "step_rowmajor_noalloc state")
    _check_param_list(table, grads, F32, "step_rowmajor_noalloc grads")
    _check(lib.fp8z1_step_rowmajor_noalloc(table.handle, C.byref(hp), _ptr(d_state), _ptr_list(grads), _ptr(master),
                                           _ptr(m), _ptr(v), _ptr(fp8), _ptr(scales), _stream(stream)),
           "fp8z1_step_rowmajor_noalloc")


def fp8z1_unfold(table: Table, folded, dtype: int, scales, dsts: Sequence, dst_scales: Optional[Sequence] = None,
                 stream=None) -> None:
    n = table.shard_slots
    _need(folded, n * 16384 * (4 if dtype == F32 else 1), "unfold folded")
    if scales is not None:
        _need(scales, n * 4, "unfold scales")
    _check_param_list(table, dsts, dtype, "unfold dst")
    if dst_scales is not None and scales is not None:
        _check_param_list(table, dst_scales, F32, "unfold dst_scales", scales=True)
    dsc = _ptr_list(dst_scales) if dst_scales is not None else None
    _check(lib.fp8z1_unfold(table.handle, _ptr(folded), dtype, _ptr(scales), _ptr_list(dsts), dsc, _stream(stream)),
           "fp8z1_unfold")


def fp8z1_state_read(d_state, stream=None) -> dict:
    out = State()
    _check(lib.fp8z1_state_read(_ptr(d_state), C.byref(out), _stream(stream)), "fp8z1_state_read")
    return out.as_dict()


def fp8z1_state_write(d_state, state: dict, stream=None) -> None:
    s = State(**{k: state[k] for k, _ in State._fields_})
    _check(lib.fp8z1_state_write(_ptr(d_state), C.byref(s), _stream(stream)), "fp8z1_state_write")


def fp8z1_encode_e4m3(x, out, stream=None) -> None:
    import torch
    _need(x, x.numel() * 4, "encode input", torch.float32)
    _need(out, x.numel(), "encode output", torch.uint8)
    _check(lib.fp8z1_encode_e4m3(_ptr(x), _ptr(out), x.numel(), _stream(stream)), "fp8z1_encode_e4m3")


def fp8z1_dequantize(codes, scales, shape, out_dtype: int, out, stream=None) -> None:
    import torch
    e, r, c = (int(x) for x in shape)
    _need(codes, e * r * c, "dequantize codes", torch.uint8)
    _need(scales, e * (-(-r // 128)) * (-(-c // 128)) * 4, "dequantize scales", torch.float32)
    _need(out, e * r * c * (4 if out_dtype == F32 else 2), "dequantize out",
          torch.float32 if out_dtype == F32 else torch.bfloat16)
    _check(lib.fp8z1_dequantize(_ptr(codes), _ptr(scales), e, r, c, out_dtype, _ptr(out), _stream(stream)),
           "fp8z1_dequantize")


def fp8z1_probe_copy(src, dst, spread: int = 1, stream=None) -> None:
    n = src.numel() * src.element_size()
    _need(dst, n, "probe_copy dst")
    _check(lib.fp8z1_probe_copy(_ptr(src), _ptr(dst), n, spread, _stream(stream)), "fp8z1_probe_copy")


def fp8z1_probe_update_pattern(g, p, m, v, codes, nslots: int, parts: int = 1, stream=None) -> None:
    for name, x in (("g", g), ("p", p), ("m", m), ("v", v)):
        _need(x, nslots * 16384 * 4, f"probe_update_pattern {name}")
    _need(codes, nslots * 16384, "probe_update_pattern codes")
    _check(lib.fp8z1_probe_update_pattern(_ptr(g), _ptr(p), _ptr(m), _ptr(v), _ptr(codes), nslots, parts,
                                          _stream(stream)), "fp8z1_probe_update_pattern")
