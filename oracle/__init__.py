"""CPU oracle for the paged, quantized KV cache: cache write + paged decode attention.

TEST INFRASTRUCTURE. A plain, slow, obviously correct fp64 NumPy implementation of what
the hot path computes, written from the pages' description and sharing no code with the
HIP path. Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import,
call or execute anything in this package; the product path never does.

Modules:
  formats    - E4M3FN / E2M1 / fp16 / bf16 encoders and decoders from their definitions
  cache      - pool layout, cache-write replay (copy, FP8, FP4 + outlier calibration),
               dequantization and block-table gather
  attention  - exact softmax decode, partition split and log-sum-exp merge
  blocks     - whole-block copies within a pool and between pools (copy on write, swap)

Parity status: every function is pinned by a `-m "not gpu"` test against closed forms,
format tables, library routines or brute force, except the FP4 calibration granularity
(which tokens a block's outlier set is computed over), a reading of the pages that is
checked only for self-consistency: parity unpinned for that choice.
"""
from . import attention, blocks, cache, formats  # noqa: F401
