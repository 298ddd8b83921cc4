"""MI355X (gfx950) block-restricted bidirectional selective scan.

Thin Python binding of libbdssm.so (C ABI in include/bdssm.h).  Every step of
the scan runs in the library's HIP kernels; this module only checks torch
tensors, allocates the caller-side workspace and passes raw device pointers
and the current HIP stream.  There is no CPU fallback: if the library is
missing, importing the binding functions raises.
"""
from .bdssm import (  # noqa: F401
    BdssmError, load, version, status_str, workspace_bytes,
    prefill, prefill_noalloc, block_step, commit, train_scan, train_scan_blocks, full_scan,
    train_scan_bwd, train_scan_blocks_bwd, bind_block_step, bind_commit, BoundCall,
    OP_PREFILL, OP_TRAIN, OP_FULL, OP_TRAIN_BWD, OP_BLOCKS_BWD, OP_TRAIN_BWD_REV, OP_BLOCKS_BWD_REV,
    F32, BF16, LIB_PATH, EXPORTS,
)
