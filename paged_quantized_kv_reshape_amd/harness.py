"""Device-side driver of one workload through libpa (tests, smoke check and bench).

Uploads a workload's inputs to HBM, derives FP8 scales with pa_fp8_head_scales, replays
its cache-write calls with pa_cache_write and runs pa_decode (+ pa_merge when split).
Everything that computes runs in libpa; torch only holds memory and orders the stream.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B

_TORCH_ACT = {"bf16": torch.bfloat16, "f16": torch.float16}


def _dev_bits(a: np.ndarray, act: str, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.to(device).view(_TORCH_ACT[act])


class DeviceRun:
    """fp4_calibration: "block" (each block's outlier set from its first write) or
    "sequence" (one set per sequence from its first 512-token prefill chunk, computed on
    the device with pa_fp4_sequence_outliers; writes go through
    pa_cache_write_seq_outliers)."""

    SEQ_CHUNK = 512

    def __init__(self, w, device="cuda", partition_size=None, fill=0xA5, pool_copies=1,
                 fp4_calibration="block", waves=None):
        assert fp4_calibration in ("block", "sequence")
        assert fp4_calibration == "block" or w.kv == "fp4"
        self.w = w
        self.waves = waves  # decode waves per workgroup (None: the library's choice)
        self.fp4_calibration = fp4_calibration
        self.device = device
        self.ps = w.partition_size if partition_size is None else partition_size
        self.q = _dev_bits(w.q, w.act, device)
        self.k_rows = _dev_bits(w.k_rows, w.act, device)
        self.v_rows = _dev_bits(w.v_rows, w.act, device)
        self.block_tables = torch.from_numpy(w.block_tables).to(device)
        self.context_lens = torch.from_numpy(w.context_lens.astype(np.int32)).to(device)
        self.dev_err = torch.zeros(1, dtype=torch.int32, device=device)
        self.k_scale = self.v_scale = None
        if w.kv in B.HEAD_SCALED:
            self.k_scale = torch.empty(w.num_kv_heads, dtype=torch.float32, device=device)
            self.v_scale = torch.empty(w.num_kv_heads, dtype=torch.float32, device=device)
            B.pa_fp8_head_scales(self.k_rows, self.k_scale, w.kv)
            B.pa_fp8_head_scales(self.v_rows, self.v_scale, w.kv)
        self.pools = [B.KVPool(w.kv, w.num_blocks, w.num_kv_heads, w.head_dim, device=device,
                               fill=fill, k_scale=self.k_scale, v_scale=self.v_scale)
                      for _ in range(pool_copies)]
        self.pool = self.pools[0]
        sc = w.step_call
        idx = torch.from_numpy(sc.rows).to(device)
        self.step_k = self.k_rows.index_select(0, idx).contiguous()
        self.step_v = self.v_rows.index_select(0, idx).contiguous()
        self.step_slots = torch.from_numpy(sc.slots).to(device)
        self.seq_records = None
        if fp4_calibration == "sequence":
            n = np.minimum(self.SEQ_CHUNK, np.maximum(w.context_lens.astype(np.int64) - 1, 0))
            rows = np.concatenate([w.seq_start[s] + np.arange(n[s]) for s in range(w.num_seqs)])
            starts = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
            idx = torch.from_numpy(rows.astype(np.int64)).to(device)
            self.seq_records = torch.empty((w.num_seqs, 2, w.num_kv_heads, 16), dtype=torch.uint8,
                                           device=device)
            B.pa_fp4_sequence_outliers(self.k_rows.index_select(0, idx),
                                       self.v_rows.index_select(0, idx),
                                       torch.from_numpy(starts).to(device), self.seq_records,
                                       self.dev_err)
            self.step_seq = self._token_seq(sc.rows)
        S, Hq, D = w.q.shape
        self.out = torch.empty((S, Hq, D), dtype=torch.float32, device=device)
        self.lse = torch.empty((S, Hq), dtype=torch.float32, device=device)
        self.part_out = self.part_lse = None
        if self.ps:
            P = B.max_partitions(w.max_blocks_per_seq, self.ps)
            self.part_out = torch.empty((S, Hq, P, D), dtype=torch.float32, device=device)
            self.part_lse = torch.empty((S, Hq, P), dtype=torch.float32, device=device)

    # -- writes ---------------------------------------------------------------------
    def _token_seq(self, rows):
        ts = np.searchsorted(self.w.seq_start, rows, side="right") - 1
        return torch.from_numpy(ts.astype(np.int32)).to(self.device)

    def _write(self, pool, k, v, slots, token_seq):
        if self.seq_records is None:
            B.pa_cache_write(pool, k, v, slots, self.dev_err)
        else:
            B.pa_cache_write_seq_outliers(pool, k, v, slots, token_seq, self.seq_records,
                                          self.dev_err)

    def setup_writes(self, pool=None):
        pool = pool or self.pool
        for call in self.w.setup_calls:
            idx = torch.from_numpy(call.rows).to(self.device)
            slots = torch.from_numpy(call.slots).to(self.device)
            ts = self._token_seq(call.rows) if self.seq_records is not None else None
            self._write(pool, self.k_rows.index_select(0, idx), self.v_rows.index_select(0, idx),
                        slots, ts)

    def step_write(self, pool=None):
        self._write(pool or self.pool, self.step_k, self.step_v, self.step_slots,
                    getattr(self, "step_seq", None))

    def prepare(self):
        for p in self.pools:
            self.setup_writes(p)
            self.step_write(p)

    # -- decode ---------------------------------------------------------------------
    def decode(self, pool=None, merge=True):
        pool = pool or self.pool
        B.pa_decode(self.q, pool, self.block_tables, self.context_lens, self.w.sm_scale,
                    self.ps, out=self.out, part_out=self.part_out, part_lse=self.part_lse,
                    dev_err=self.dev_err, waves=self.waves)
        if merge:
            self.merge()

    def merge(self):
        if self.ps:
            B.pa_merge(self.part_out, self.part_lse, self.context_lens, self.ps, self.out,
                       self.lse)

    def step(self, pool=None):
        """One pass of the hot path: the step's cache write, then decode (+ merge)."""
        self.step_write(pool)
        self.decode(pool)

    @property
    def step_rows_per_seq(self) -> int:
        """n when the step writes the last n positions of every sequence, in sequence order
        (then it can run as one pa_append_decode[_n] launch), else 0."""
        w = self.w
        S = w.num_seqs
        if len(w.step_call.rows) % S:
            return 0
        n = len(w.step_call.rows) // S
        L = w.context_lens.astype(np.int64)
        if n == 0 or np.any(L < n):
            return 0
        want = (w.seq_start[:, None] + L[:, None] - n + np.arange(n)[None, :]).reshape(-1)
        return n if np.array_equal(w.step_call.rows, want) else 0

    @property
    def can_append(self) -> bool:
        """The step can run as one launch that writes and decodes: it writes the last n
        positions of every sequence (n = 1 in a 4-bit pool, whose per-block calibration
        takes a block's first-write rows; the per-sequence mode writes through its own entry
        point)."""
        n = self.step_rows_per_seq
        return self.seq_records is None and (n == 1 or (n > 1 and self.w.kv != "fp4"))

    def append_decode(self, pool=None, merge=True):
        n = self.step_rows_per_seq
        if n == 1:
            B.pa_append_decode(self.q, pool or self.pool, self.step_k, self.step_v,
                               self.block_tables, self.context_lens, self.w.sm_scale, self.ps,
                               out=self.out, part_out=self.part_out, part_lse=self.part_lse,
                               dev_err=self.dev_err, waves=self.waves)
        else:
            S = self.w.num_seqs
            B.pa_append_decode_n(self.q, pool or self.pool,
                                 self.step_k.view(S, n, *self.step_k.shape[1:]),
                                 self.step_v.view(S, n, *self.step_v.shape[1:]),
                                 self.block_tables, self.context_lens, self.w.sm_scale, self.ps,
                                 out=self.out, part_out=self.part_out, part_lse=self.part_lse,
                                 dev_err=self.dev_err, waves=self.waves)
        if merge:
            self.merge()

    def step_fused(self, pool=None):
        """The same step in one launch (+ merge): each sequence's new row is written by the
        decode workgroup that reads it."""
        self.append_decode(pool)

    def gather_probe(self, pool=None, sink=None):
        """The decode's launch with its tile reads only (pa_gather_probe)."""
        if sink is None:
            if getattr(self, "probe_sink", None) is None:
                self.probe_sink = torch.zeros(B.PROBE_SINK_WORDS, dtype=torch.int32,
                                              device=self.device)
            sink = self.probe_sink
        B.pa_gather_probe(pool or self.pool, self.w.num_q_heads, self.block_tables,
                          self.context_lens, self.ps, sink, self.dev_err, waves=self.waves)

    def device_error(self) -> int:
        return B.pa_read_device_error(self.dev_err)


# ---------------------------------------------------------------------------------
# Algorithmic bytes: what the method itself must move, not what a kernel happens to fetch.
# ---------------------------------------------------------------------------------
_KV_ELEM_BITS = {"f16": 16, "bf16": 16, "fp8": 8, "fp4": 4, "bf8": 8, "fp8t": 8, "bf8t": 8}


def outlier_counts(run) -> dict:
    """FP4 only: total outlier channels over all written (block, kv head) records, K and V
    (read from the device pool's records; 0xFF = never written counts 0)."""
    out = {}
    for side in ("k", "v"):
        rec = run.pool.fp4_records(side)[:, :, 0].to(torch.int32)
        out[side] = int(torch.where(rec == 0xFF, torch.zeros_like(rec), rec).sum().item())
    return out


def decode_bytes(w, outliers=None) -> dict:
    """Algorithmic bytes of one pa_decode (+ merge) over workload w: every stored K/V byte
    of every attended token read once (codes; FP4 also the per-token scales, the 16-byte
    record of each (block, kv head) and its fp16 outlier values), the block-table entries
    of the attended blocks, the context lengths, q (16-bit) and out (fp32)."""
    L = w.context_lens.astype(np.int64)
    hkv, d, S, hq = w.num_kv_heads, w.head_dim, w.num_seqs, w.num_q_heads
    tok = int(L.sum())
    blocks = int((-(-L // 16)).sum())
    kv = 2 * tok * hkv * d * _KV_ELEM_BITS[w.kv] // 8
    extra = 0
    if w.kv == "fp4":
        extra += 2 * tok * hkv * 4            # per-token fp32 scales, K and V
        extra += 2 * blocks * hkv * 16        # outlier records
        if outliers is not None:              # fp16 values of every outlier channel
            extra += (outliers["k"] + outliers["v"]) * 16 * 2
    if w.kv in ("fp8", "bf8"):
        extra += 2 * hkv * 4                  # per-head scales
    if w.kv in ("fp8t", "bf8t"):
        extra += 2 * tok * hkv * 4            # per-token fp32 scales, K and V
    meta = blocks * 4 + S * 4
    io = S * hq * d * 2 + S * hq * d * 4
    return {"kv": kv + extra, "meta": meta, "io": io, "total": kv + extra + meta + io,
            "tokens": tok, "blocks": blocks}


def write_bytes(w, num_tokens: int) -> int:
    """Algorithmic bytes of one pa_cache_write of num_tokens rows: read the new K and V
    rows and their slots, store the encoded rows (FP4 also the per-token scales)."""
    hkv, d = w.num_kv_heads, w.head_dim
    rd = num_tokens * (2 * hkv * d * 2 + 8)
    wr = 2 * num_tokens * hkv * d * _KV_ELEM_BITS[w.kv] // 8
    if w.kv in ("fp4", "fp8t", "bf8t"):
        wr += 2 * num_tokens * hkv * 4
    return rd + wr
