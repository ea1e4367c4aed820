"""Python binding of libfp8z1 (the blockwise-FP8 ZeRO-1 shard step for MI355X).

Argument marshalling only: every step of the path runs in the HIP library.
The functions keep the C names of ``include/fp8z1.h``; tensors are passed
as device pointers, streams as ``torch.cuda.current_stream().cuda_stream``.
Importing this package loads the library and raises if it is not built.
"""
from ._lib import (  # noqa: F401
    ALL_RANKS, BF16, E4M3, F32, NOALLOC_MAX_SLOTS, SCALE_AMAX, SCALE_POW2, SPLIT_BLOCK, SPLIT_PARAM, STAT_PARTS,
    BLOCK_ENTRY_DTYPE, Fp8z1Error, Hparams, State, Table,
    fp8z1_build_table, fp8z1_dequantize, fp8z1_encode_e4m3, fp8z1_fold, fp8z1_state_init, fp8z1_state_read, fp8z1_state_write,
    fp8z1_shard_sumsq, fp8z1_step, fp8z1_step_rowmajor, fp8z1_step_rowmajor_noalloc, fp8z1_step_workspace_bytes,
    fp8z1_unfold, fp8z1_probe_copy,
    fp8z1_probe_update_pattern, lib, lib_path,
)
