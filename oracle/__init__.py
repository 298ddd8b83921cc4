"""fp64 CPU oracle of the block-restricted bidirectional selective scan.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only permitted users.  The GPU library
does not import, link or call anything here, and nothing here calls the GPU
library.

The arithmetic lives in ``bdssm_oracle.c`` (plain C, fp64, one sequential loop
over tokens per (batch, channel) row); this module only marshals numpy arrays
through ctypes.  Which passage of the pages each step follows is stated in the
C file's header.
"""
from .oracle import (  # noqa: F401
    build, load, scan, prefill, block_step, commit, train_scan, full_scan, train_blocks,
    scan_bwd, F32, BF16, F64, num_threads,
)
