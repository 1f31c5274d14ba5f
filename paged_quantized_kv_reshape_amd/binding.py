"""Thin ctypes binding of libpa (include/pa.h), with the C entry points' names.

Argument marshalling only: torch tensors supply device memory and the current HIP stream,
and every step of the hot path runs in libpa's gfx950 kernels. There is no fallback: if
libpa.so is missing or a call is rejected, this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")
_lib = None

KV_DTYPES = {"f16": 0, "bf16": 1, "fp8": 2, "fp4": 3, "bf8": 4, "fp8t": 5, "bf8t": 6}
# pool formats with one fp32 scale per kv head (inputs: k_scale / v_scale)
HEAD_SCALED = ("fp8", "bf8")
ACT_DTYPES = {torch.float16: 0, torch.bfloat16: 1}
BLOCK_SIZE = 16
DEVERR_BITS = {1: "bad block id", 2: "bad slot", 4: "bad context length",
               8: "read of an uncalibrated FP4 block"}
PROBE_SINK_WORDS = 1024  # pa_gather_probe's sink: uint32 [1024]


class PAError(RuntimeError):
    """A libpa call returned a non-zero pa_status."""

    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {lib().pa_status_string(status).decode()} (status {status})")
        self.status = status


class pa_kv_pool(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("k_out_val", ctypes.c_void_p), ("v_out_val", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
    ]


class pa_launch_options(ctypes.Structure):
    _fields_ = [("decode_waves", ctypes.c_int32), ("prefill_col_tiles", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 6)]


def _opts(decode_waves=None, prefill_col_tiles=None):
    """A pa_launch_options for the _ex entry points, or None (the library's choice)."""
    if decode_waves is None and prefill_col_tiles is None:
        return None
    o = pa_launch_options()
    o.decode_waves = int(decode_waves or 0)
    o.prefill_col_tiles = int(prefill_col_tiles or 0)
    return ctypes.byref(o)


def fp4_tile_bytes(head_dim: int) -> int:
    """PA_FP4_TILE_BYTES of include/pa.h."""
    return (8 * head_dim + 112 + 127) // 128 * 128


def fp4_record_offset(head_dim: int) -> int:
    """PA_FP4_RECORD_OFF of include/pa.h."""
    return 8 * head_dim + 64


def lib():
    """Load libpa.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"libpa.so not found at {_LIB_PATH}; build it with "
                               "`python -m paged_quantized_kv_reshape_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        pool_p = ctypes.POINTER(pa_kv_pool)
        sig = {
            "pa_pool_layout": (ctypes.c_int, [i32, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]),
            "pa_outlier_capacity": (ctypes.c_int, [i32]),
            "pa_cache_write": (ctypes.c_int, [pool_p, vp, vp, i32, i32, vp, vp, vp]),
            "pa_fp8_head_scales": (ctypes.c_int, [vp, i32, i32, i64, i32, i32, vp, vp]),
            "pa_reset_blocks": (ctypes.c_int, [pool_p, vp, i32, vp]),
            "pa_decode": (ctypes.c_int, [vp, i32, i32, i32, pool_p, vp, i32, vp, f32, i32, vp, vp,
                                         vp, vp, vp]),
            "pa_prefill": (ctypes.c_int, [vp, i32, i32, i32, i32, vp, i32, pool_p, vp, i32, vp,
                                          f32, vp, vp, vp]),
            "pa_merge": (ctypes.c_int, [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp]),
            "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "pa_read_device_error": (ctypes.c_int, [vp, vp, vp]),
            "pa_copy_blocks": (ctypes.c_int, [pool_p, pool_p, vp, i32, vp, vp]),
            "pa_append_decode": (ctypes.c_int, [vp, i32, i32, i32, pool_p, vp, vp, vp, i32, vp,
                                                f32, i32, vp, vp, vp, vp, vp]),
            "pa_fp4_sequence_outliers": (ctypes.c_int, [vp, vp, i32, i64, i32, i32, vp, i32, vp,
                                                        vp, vp]),
            "pa_cache_write_seq_outliers": (ctypes.c_int, [pool_p, vp, vp, i32, i32, vp, vp, vp,
                                                           i32, vp, vp]),
            "pa_allocator_create": (ctypes.c_int, [i32, ctypes.POINTER(vp)]),
            "pa_allocator_destroy": (ctypes.c_int, [vp]),
            "pa_allocator_alloc": (ctypes.c_int, [vp, i32, vp]),
            "pa_allocator_share": (ctypes.c_int, [vp, vp, i32]),
            "pa_allocator_release": (ctypes.c_int, [vp, vp, i32, vp, vp]),
            "pa_allocator_writable": (ctypes.c_int, [vp, i32, ctypes.POINTER(i32)]),
            "pa_allocator_refcount": (ctypes.c_int, [vp, i32]),
            "pa_allocator_num_free": (ctypes.c_int, [vp]),
            "pa_decode_ex": (ctypes.c_int, [vp, i32, i32, i32, pool_p, vp, i32, vp, f32, i32, vp,
                                            vp, vp, vp, vp, vp]),
            "pa_append_decode_ex": (ctypes.c_int, [vp, i32, i32, i32, pool_p, vp, vp, vp, i32,
                                                   vp, f32, i32, vp, vp, vp, vp, vp, vp]),
            "pa_append_decode_n": (ctypes.c_int, [vp, i32, i32, i32, pool_p, vp, vp, i32, vp,
                                                  i32, vp, f32, i32, vp, vp, vp, vp, vp, vp]),
            "pa_prefill_ex": (ctypes.c_int, [vp, i32, i32, i32, i32, vp, i32, pool_p, vp, i32,
                                             vp, f32, vp, vp, vp, vp]),
            "pa_gather_probe": (ctypes.c_int, [i32, i32, pool_p, vp, i32, vp, i32, vp, vp, vp,
                                               vp]),
            "pa_decode_split_static": (ctypes.c_int, [vp, i32, i32, i32, pool_p, vp, i32, vp,
                                                      f32, i32, vp, vp, vp, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _check(fn, status):
    if status != 0:
        raise PAError(fn, status)


def pa_pool_layout(kv_dtype: str, num_blocks: int, num_kv_heads: int, head_dim: int):
    out = (ctypes.c_size_t * 4)()
    _check("pa_pool_layout", lib().pa_pool_layout(KV_DTYPES[kv_dtype], num_blocks, num_kv_heads,
                                                  head_dim, out))
    return list(out)


def pa_outlier_capacity(head_dim: int) -> int:
    c = lib().pa_outlier_capacity(head_dim)
    if c < 0:
        raise PAError("pa_outlier_capacity", c)
    return c


class KVPool:
    """Arrays of one paged pool (caller-owned memory, as the ABI requires).

    `fill` is the byte every array starts with; FP4 outlier records are then set to 0xFF
    (never written): with pa_reset_blocks on the GPU, or directly for a pool in pinned
    host memory (device="cpu", the destination of swaps). Per-head FP8 pools on the GPU
    need k_scale / v_scale [Hkv] fp32 device tensors."""

    NAMES = ["k", "v", "k_out_val", "v_out_val"]

    def __init__(self, kv_dtype, num_blocks, num_kv_heads, head_dim, device="cuda", fill=0,
                 k_scale=None, v_scale=None):
        self.kv_dtype, self.num_blocks = kv_dtype, num_blocks
        self.num_kv_heads, self.head_dim = num_kv_heads, head_dim
        sizes = pa_pool_layout(kv_dtype, num_blocks, num_kv_heads, head_dim)
        self.host = torch.device(device).type == "cpu"
        self.bytes = {}
        for name, n in zip(self.NAMES, sizes):
            if n:
                if self.host:  # pinned (hipHostMalloc), so the GPU can reach it in place
                    t = torch.empty((n,), dtype=torch.uint8, pin_memory=True)
                    self.bytes[name] = t.fill_(fill)
                else:
                    self.bytes[name] = torch.full((n,), fill, dtype=torch.uint8, device=device)
        self.k_scale, self.v_scale = k_scale, v_scale
        if kv_dtype in HEAD_SCALED and not self.host and (k_scale is None or v_scale is None):
            raise ValueError(f"a {kv_dtype} pool needs k_scale and v_scale")
        if kv_dtype == "fp4":
            if self.host:
                for side in ("k", "v"):
                    self.fp4_records(side).fill_(0xFF)
            else:
                pa_reset_blocks(self, torch.arange(num_blocks, dtype=torch.int32, device=device))

    def fp4_records(self, side: str):
        """FP4 only: the 16-byte outlier records [NB, Hkv, 16] (a view of the k or v tiles)."""
        t = self.bytes[side].view(self.num_blocks, self.num_kv_heads,
                                  fp4_tile_bytes(self.head_dim))
        o = fp4_record_offset(self.head_dim)
        return t[:, :, o:o + 16]

    def struct(self) -> pa_kv_pool:
        s = pa_kv_pool()
        s.dtype = KV_DTYPES[self.kv_dtype]
        s.num_blocks, s.block_size = self.num_blocks, BLOCK_SIZE
        s.num_kv_heads, s.head_dim = self.num_kv_heads, self.head_dim
        for name in self.NAMES:
            setattr(s, name, _ptr(self.bytes.get(name)))
        s.k_scale, s.v_scale = _ptr(self.k_scale), _ptr(self.v_scale)
        return s

    def numpy(self) -> dict:
        """Host copies of the raw pool bytes, keyed like the arrays of the ABI."""
        return {n: t.cpu().numpy() for n, t in self.bytes.items()}


def pa_cache_write(pool: KVPool, k_new, v_new, slot_mapping, dev_err=None):
    assert k_new.dtype in ACT_DTYPES and v_new.dtype == k_new.dtype
    assert slot_mapping.dtype == torch.int64
    T = k_new.shape[0]
    s = pool.struct()
    _check("pa_cache_write", lib().pa_cache_write(
        ctypes.byref(s), _ptr(k_new), _ptr(v_new), ACT_DTYPES[k_new.dtype], T,
        _ptr(slot_mapping), _ptr(dev_err), _stream()))


def pa_fp4_sequence_outliers(k_rows, v_rows, row_start, seq_records, dev_err=None):
    """k_rows, v_rows [R, Hkv, 128] fp16/bf16; row_start [S + 1] int32; seq_records
    [S, 2, Hkv, 16] uint8 (written)."""
    assert k_rows.dtype in ACT_DTYPES and v_rows.dtype == k_rows.dtype
    assert k_rows.shape == v_rows.shape and row_start.dtype == torch.int32
    assert seq_records.dtype == torch.uint8
    S = row_start.numel() - 1
    assert tuple(seq_records.shape) == (S, 2, k_rows.shape[1], 16)
    _check("pa_fp4_sequence_outliers", lib().pa_fp4_sequence_outliers(
        _ptr(k_rows), _ptr(v_rows), ACT_DTYPES[k_rows.dtype], k_rows.shape[0], k_rows.shape[1],
        k_rows.shape[2], _ptr(row_start), S, _ptr(seq_records), _ptr(dev_err), _stream()))


def pa_cache_write_seq_outliers(pool: KVPool, k_new, v_new, slot_mapping, token_seq,
                                seq_records, dev_err=None):
    assert k_new.dtype in ACT_DTYPES and v_new.dtype == k_new.dtype
    assert slot_mapping.dtype == torch.int64 and token_seq.dtype == torch.int32
    assert seq_records.dtype == torch.uint8
    s = pool.struct()
    _check("pa_cache_write_seq_outliers", lib().pa_cache_write_seq_outliers(
        ctypes.byref(s), _ptr(k_new), _ptr(v_new), ACT_DTYPES[k_new.dtype], k_new.shape[0],
        _ptr(slot_mapping), _ptr(token_seq), _ptr(seq_records), seq_records.shape[0],
        _ptr(dev_err), _stream()))


def pa_fp8_head_scales(x, scale_out, kv_dtype="fp8"):
    """x [rows, Hkv, D] fp16/bf16 -> scale_out [Hkv] fp32 (overwritten) for a pool of
    kv_dtype "fp8" (E4M3, absmax / 448) or "bf8" (E5M2, absmax / 57344)."""
    assert x.dtype in ACT_DTYPES and scale_out.dtype == torch.float32
    _check("pa_fp8_head_scales", lib().pa_fp8_head_scales(
        _ptr(x), ACT_DTYPES[x.dtype], KV_DTYPES[kv_dtype], x.shape[0], x.shape[1], x.shape[2],
        _ptr(scale_out), _stream()))


def pa_reset_blocks(pool: KVPool, block_ids):
    assert block_ids.dtype == torch.int32
    s = pool.struct()
    _check("pa_reset_blocks", lib().pa_reset_blocks(ctypes.byref(s), _ptr(block_ids),
                                                    block_ids.numel(), _stream()))


def pa_copy_blocks(src: KVPool, dst: KVPool, pairs, dev_err=None):
    """pairs [n, 2] int32 (source block of src, destination block of dst), on the GPU or
    in pinned host memory; src may be dst (copy on write) or either may be a host pool
    (swap)."""
    assert pairs.dtype == torch.int32 and pairs.dim() == 2 and pairs.shape[1] == 2
    assert pairs.is_contiguous()
    s, d = src.struct(), dst.struct()
    _check("pa_copy_blocks", lib().pa_copy_blocks(ctypes.byref(s), ctypes.byref(d),
                                                  _ptr(pairs), pairs.shape[0], _ptr(dev_err),
                                                  _stream()))


class BlockAllocator:
    """The library's host-side reference-counted block allocator (pa_allocator_*)."""

    def __init__(self, num_blocks: int):
        h = ctypes.c_void_p()
        _check("pa_allocator_create", lib().pa_allocator_create(num_blocks, ctypes.byref(h)))
        self._h = h
        self.num_blocks = num_blocks

    def close(self):
        if self._h:
            lib().pa_allocator_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def _ids(ids):
        arr = (ctypes.c_int32 * max(len(ids), 1))(*[int(i) for i in ids])
        return arr, len(ids)

    def alloc(self, n: int) -> list:
        out = (ctypes.c_int32 * max(n, 1))()
        _check("pa_allocator_alloc", lib().pa_allocator_alloc(self._h, n, out))
        return list(out)[:n]

    def share(self, ids):
        arr, n = self._ids(ids)
        _check("pa_allocator_share", lib().pa_allocator_share(self._h, arr, n))

    def release(self, ids) -> list:
        """Drop one reference per listed id; returns the ids that became free."""
        arr, n = self._ids(ids)
        freed = (ctypes.c_int32 * max(n, 1))()
        k = ctypes.c_int32()
        _check("pa_allocator_release", lib().pa_allocator_release(self._h, arr, n, freed,
                                                                 ctypes.byref(k)))
        return list(freed)[:k.value]

    def writable(self, block_id: int):
        """(id to write into, whether the caller must copy block_id there first)."""
        out = ctypes.c_int32()
        r = lib().pa_allocator_writable(self._h, block_id, ctypes.byref(out))
        if r < 0:
            raise PAError("pa_allocator_writable", r)
        return out.value, r == 1

    def refcount(self, block_id: int) -> int:
        r = lib().pa_allocator_refcount(self._h, block_id)
        if r < 0:
            raise PAError("pa_allocator_refcount", r)
        return r

    @property
    def num_free(self) -> int:
        return lib().pa_allocator_num_free(self._h)


def max_partitions(max_blocks_per_seq: int, partition_size: int) -> int:
    return -(-max_blocks_per_seq * BLOCK_SIZE // partition_size) if partition_size else 1


def pa_decode(q, pool: KVPool, block_tables, context_lens, sm_scale, partition_size=0, out=None,
              part_out=None, part_lse=None, dev_err=None, waves=None):
    """q [S, Hq, D]; block_tables [S, MB] int32; context_lens [S] int32. With
    partition_size = 0 fills out [S, Hq, D] fp32; otherwise part_out / part_lse. waves
    (1, 2, 4, 8) fixes the waves per workgroup (pa_decode_ex), else the library picks."""
    assert q.dtype in ACT_DTYPES and block_tables.dtype == torch.int32
    assert context_lens.dtype == torch.int32
    S, Hq, _ = q.shape
    s = pool.struct()
    args = (_ptr(q), ACT_DTYPES[q.dtype], S, Hq, ctypes.byref(s), _ptr(block_tables),
            block_tables.shape[1], _ptr(context_lens), float(sm_scale), partition_size, _ptr(out),
            _ptr(part_out), _ptr(part_lse), _ptr(dev_err))
    if waves is None:
        _check("pa_decode", lib().pa_decode(*args, _stream()))
    else:
        _check("pa_decode_ex", lib().pa_decode_ex(*args, _opts(waves), _stream()))


def pa_append_decode(q, pool: KVPool, k_new, v_new, block_tables, context_lens, sm_scale,
                     partition_size=0, out=None, part_out=None, part_lse=None, dev_err=None,
                     waves=None):
    """pa_decode after writing each sequence's new row k_new[s] / v_new[s] ([S, Hkv, D],
    q's dtype) at its last position, in one launch (every pool format)."""
    assert q.dtype in ACT_DTYPES and k_new.dtype == q.dtype and v_new.dtype == q.dtype
    assert block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32
    assert k_new.is_contiguous() and v_new.is_contiguous()
    S, Hq, _ = q.shape
    s = pool.struct()
    args = (_ptr(q), ACT_DTYPES[q.dtype], S, Hq, ctypes.byref(s), _ptr(k_new), _ptr(v_new),
            _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), float(sm_scale),
            partition_size, _ptr(out), _ptr(part_out), _ptr(part_lse), _ptr(dev_err))
    if waves is None:
        _check("pa_append_decode", lib().pa_append_decode(*args, _stream()))
    else:
        _check("pa_append_decode_ex", lib().pa_append_decode_ex(*args, _opts(waves), _stream()))


def pa_append_decode_n(q, pool: KVPool, k_new, v_new, block_tables, context_lens, sm_scale,
                       partition_size=0, out=None, part_out=None, part_lse=None, dev_err=None,
                       waves=None):
    """pa_decode after writing each sequence's n new rows k_new[s, i] / v_new[s, i]
    ([S, n, Hkv, D], q's dtype) at its positions L_s - n + i, in one launch (16-bit and FP8
    pools; FP4 pools take n = 1)."""
    assert q.dtype in ACT_DTYPES and k_new.dtype == q.dtype and v_new.dtype == q.dtype
    assert block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32
    assert k_new.is_contiguous() and v_new.is_contiguous() and k_new.dim() == 4
    S, Hq, _ = q.shape
    assert k_new.shape[0] == S and v_new.shape == k_new.shape
    s = pool.struct()
    _check("pa_append_decode_n", lib().pa_append_decode_n(
        _ptr(q), ACT_DTYPES[q.dtype], S, Hq, ctypes.byref(s), _ptr(k_new), _ptr(v_new),
        int(k_new.shape[1]), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        float(sm_scale), partition_size, _ptr(out), _ptr(part_out), _ptr(part_lse),
        _ptr(dev_err), _opts(waves), _stream()))


def pa_prefill(q, query_start, max_query_len, pool: KVPool, block_tables, context_lens,
               sm_scale, out, dev_err=None, col_tiles=None):
    """q [T, Hq, D]; query_start [S + 1] int32 (sequence s owns rows query_start[s] ..
    query_start[s + 1] - 1, its last positions); fills out [T, Hq, D] fp32."""
    assert q.dtype in ACT_DTYPES and block_tables.dtype == torch.int32
    assert context_lens.dtype == torch.int32 and query_start.dtype == torch.int32
    S = context_lens.shape[0]
    assert query_start.shape[0] == S + 1
    T, Hq, _ = q.shape
    assert out.shape[0] == T
    s = pool.struct()
    args = (_ptr(q), ACT_DTYPES[q.dtype], S, Hq, T, _ptr(query_start), int(max_query_len),
            ctypes.byref(s), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
            float(sm_scale), _ptr(out), _ptr(dev_err))
    if col_tiles is None:
        _check("pa_prefill", lib().pa_prefill(*args, _stream()))
    else:
        _check("pa_prefill_ex", lib().pa_prefill_ex(*args, _opts(prefill_col_tiles=col_tiles),
                                                    _stream()))


def pa_gather_probe(pool: KVPool, num_q_heads, block_tables, context_lens, partition_size,
                    sink, dev_err=None, waves=None):
    """The decode's launch and tile reads with no arithmetic (a bandwidth ceiling); sink
    [1024] uint32 device tensor."""
    assert block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32
    assert sink.dtype == torch.int32 and sink.numel() >= PROBE_SINK_WORDS
    s = pool.struct()
    _check("pa_gather_probe", lib().pa_gather_probe(
        context_lens.shape[0], num_q_heads, ctypes.byref(s), _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), partition_size, _ptr(sink), _ptr(dev_err),
        _opts(waves), _stream()))


def pa_decode_split_static(q, pool: KVPool, block_tables, context_lens, sm_scale,
                           partition_size, out, lse_out=None, dev_err=None):
    """Split decode + merge into out [S, Hq, D] (lse_out [S, Hq] optional), the partials
    in the library's static device scratch: no allocation of any kind."""
    assert q.dtype in ACT_DTYPES and block_tables.dtype == torch.int32
    assert context_lens.dtype == torch.int32
    S, Hq, _ = q.shape
    s = pool.struct()
    _check("pa_decode_split_static", lib().pa_decode_split_static(
        _ptr(q), ACT_DTYPES[q.dtype], S, Hq, ctypes.byref(s), _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), float(sm_scale), partition_size, _ptr(out),
        _ptr(lse_out), _ptr(dev_err), _stream()))


def pa_merge(part_out, part_lse, context_lens, partition_size, out, lse_out=None):
    S, Hq, P, D = part_out.shape
    _check("pa_merge", lib().pa_merge(
        _ptr(part_out), _ptr(part_lse), _ptr(context_lens), S, Hq, D, P, partition_size,
        _ptr(out), _ptr(lse_out), _stream()))


def pa_read_device_error(dev_err) -> int:
    host = ctypes.c_int32(0)
    _check("pa_read_device_error", lib().pa_read_device_error(_ptr(dev_err), ctypes.byref(host),
                                                              _stream()))
    return host.value


def describe_device_error(bits: int) -> str:
    return ", ".join(v for k, v in DEVERR_BITS.items() if bits & k) or "none"
