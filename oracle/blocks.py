"""Whole-block copies between paged pools (fp64-free: bytes only, CPU).

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg may import this package.

What the pages fix:
  * Physical KV blocks can be shared by several sequences, for beam search and parallel
    sampling, and reused across requests that share a prompt prefix (inferensys glossary
    "vLLM", PagedAttention entry and automatic prefix caching entry). A shared block that
    one of its sequences must extend is first duplicated (copy on write), which is a
    whole-block copy inside one pool.
  * Under memory pressure the engine preempts a sequence by swapping its KV blocks out to
    host RAM and back in later (inferensys glossary "vLLM", preemption and CPU offloading
    entries), which is a whole-block copy between the device pool and a pool of the same
    format in host memory.

Readings (listed in the design notes):
  * A copy moves every byte a block owns in every array of the pool: the codes, the
    per-token scales and FP4 records stored in the block's runs, and the FP4 outlier slots.
    Per-head FP8 scales belong to the (layer, head), not to a block, and are not copied.
  * A copied FP4 block carries its calibration record, so later writes into the copy
    reuse the source's outlier set (the record is part of the block's state).
  * In one call the destination ids are distinct and, within one pool, no destination is
    also a source; under that condition the order of the pairs does not matter.
"""
from __future__ import annotations

import numpy as np

from .cache import Pool


def same_geometry(a: Pool, b: Pool) -> bool:
    return (a.kind, a.num_kv_heads, a.head_dim) == (b.kind, b.num_kv_heads, b.head_dim)


def copy_blocks(src: Pool, dst: Pool, pairs) -> None:
    """For every (s, d) in pairs: block d of dst becomes a byte-for-byte copy of block s of
    src, in every array. src and dst may be the same pool."""
    assert same_geometry(src, dst), "pools of different formats or shapes"
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    if len(pairs) == 0:
        return
    s, d = pairs[:, 0], pairs[:, 1]
    assert ((s >= 0) & (s < src.num_blocks)).all() and ((d >= 0) & (d < dst.num_blocks)).all()
    assert len(np.unique(d)) == len(d), "destination blocks must be distinct"
    if src is dst:
        assert not np.isin(d, s).any(), "a destination is also a source in the same pool"
    for name, arr in src.arrays.items():
        dst.arrays[name][d] = arr[s]
