"""Paged, quantized KV cache for AMD Instinct MI355X (gfx950): cache write, paged decode,
multi-token (prefill / draft-verification) paged attention, whole-block copies (copy on
write, swap to pinned host memory) and a host-side reference-counted block allocator.

The kernels and the C ABI live in libpa.so (sources in csrc/, declarations in
include/pa.h); `binding` is a thin ctypes layer over it with the same entry-point names.
"""
from .binding import (  # noqa: F401
    BlockAllocator, KVPool, PAError, describe_device_error, lib, max_partitions, pa_append_decode,
    pa_append_decode_n, pa_cache_write,
    pa_cache_write_seq_outliers, pa_copy_blocks, pa_decode, pa_decode_split_static,
    pa_fp4_sequence_outliers,
    pa_fp8_head_scales, pa_gather_probe, pa_merge, pa_outlier_capacity, pa_pool_layout,
    pa_prefill, pa_read_device_error, pa_reset_blocks,
)
