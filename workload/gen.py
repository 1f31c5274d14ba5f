"""Seeded synthetic workloads for the paged KV cache (shared by tests, bench and smoke).

This module only draws inputs; it holds none of the method's arithmetic (no quantizer,
no scale, no attention). Both the oracle and the HIP path consume what it returns.

Shapes follow the pages' serving workloads: 16-token blocks (xonoai.com field report on
vLLM v0.7.2, "Production Configuration Snippet"), 256 concurrent 8k-token streams on the
Llama-3.1-70B 8-GPU tensor-parallel deployment (same report, "Comparative Inference Engine
Performance"; one GPU's share is 8 query heads over 1 kv head), 64k to 120k-token contexts
(dailyaiworld.com, "vLLM 0.7 Ships Unified KV Cache Compression", opening section; the
xonoai.com report's --max-model-len 131072), prefill in 512-token chunks (the dailyaiworld
engine diagram) and roughly 0.1% of activation channels carrying large outliers (the
dailyaiworld "Technical Breakdown" section). No dataset item is used: every value is drawn
here from N(0, 1).

Recipe (fixed): root = numpy SeedSequence(seed), spawned into four streams: structure, Q,
K and V. The structure stream (PCG64) draws, in order, the context lengths, the block-table
permutation and the planted outlier channels. Q, K and V rows are drawn in fixed chunks of
2^22 values rounded down to whole rows; chunk i of a tensor uses PCG64 on the i-th child of
that tensor's stream (so chunks can be drawn in parallel threads, with the same result).
Values are N(0,1) in fp32 (standard_normal, float32); planted
channels (n = max(1, round(0.001 * Hkv * D)) flattened (head, channel) pairs per tensor,
chosen without replacement, separately for K and V, fixed over tokens) are multiplied by 20
in fp32; then every value is rounded to nearest-even in the activation dtype and kept as
raw uint16 bits.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BLOCK = 16
_CHUNK = 1 << 22  # values drawn per standard_normal call (fixed: part of the recipe)


def _round_into(x32: np.ndarray, act: str, out16: np.ndarray, tmp: np.ndarray) -> None:
    """Round fp32 values to the activation dtype (nearest even) as raw bits, into out16.
    tmp is a uint32 scratch array of x32's shape (reused so no pages are faulted in)."""
    if act == "bf16":
        u = x32.view(np.uint32)
        np.right_shift(u, np.uint32(16), out=tmp)
        np.bitwise_and(tmp, np.uint32(1), out=tmp)
        np.add(tmp, u, out=tmp)
        np.add(tmp, np.uint32(0x7FFF), out=tmp)
        np.right_shift(tmp, np.uint32(16), out=tmp)
        out16[...] = tmp
    elif act == "f16":
        out16[...] = x32.astype(np.float16).view(np.uint16)
    else:
        raise ValueError(act)


def _normal_rows(stream: np.random.SeedSequence, n_rows, hkv, d, act, planted=None,
                 threads: int = 8):
    """[n_rows, hkv, d] uint16 rows of N(0,1) values drawn chunk by chunk (chunk i from
    the i-th child of `stream`), rounded to the activation dtype."""
    out = np.empty((n_rows, hkv, d), dtype=np.uint16)
    flat = out.reshape(n_rows, hkv * d)
    per = max(1, _CHUNK // (hkv * d))
    n_chunks = -(-n_rows // per)
    children = stream.spawn(n_chunks)
    rows = min(per, max(n_rows, 1))
    local = threading.local()

    def work(i):
        if not hasattr(local, "buf"):
            local.buf = np.empty((rows, hkv * d), dtype=np.float32)
            local.tmp = np.empty((rows, hkv * d), dtype=np.uint32)
        lo, hi = i * per, min(n_rows, (i + 1) * per)
        x = local.buf[:hi - lo]
        np.random.Generator(np.random.PCG64(children[i])).standard_normal(out=x, dtype=np.float32)
        if planted is not None and len(planted):
            x[:, planted] *= np.float32(20.0)
        _round_into(x, act, flat[lo:hi], local.tmp[:hi - lo])

    if n_chunks <= 1 or threads <= 1:
        for i in range(n_chunks):
            work(i)
    else:
        with ThreadPoolExecutor(min(threads, n_chunks)) as ex:
            list(ex.map(work, range(n_chunks)))
    return out


@dataclass
class WriteCall:
    rows: np.ndarray   # int64 [T] indices into Workload.k_rows / v_rows
    slots: np.ndarray  # int64 [T] physical_block * 16 + offset


@dataclass
class Workload:
    name: str
    seed: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    kv: str              # "f16" | "bf16" | "fp8" | "fp4"
    act: str             # "f16" | "bf16"
    context_lens: np.ndarray   # int32 [S]
    num_blocks: int
    block_tables: np.ndarray   # int32 [S, MB], -1 past each sequence's last block
    q: np.ndarray              # uint16 [S, Hq, D]
    k_rows: np.ndarray         # uint16 [sum L, Hkv, D], sequence-major
    v_rows: np.ndarray
    seq_start: np.ndarray      # int64 [S] first row of each sequence
    setup_calls: list = field(default_factory=list)
    step_call: WriteCall | None = None
    sm_scale: float = 0.0
    partition_size: int = 0
    planted_k: np.ndarray | None = None  # flattened (head * D + channel) indices
    planted_v: np.ndarray | None = None

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def tokens(self) -> int:
        return int(self.context_lens.astype(np.int64).sum())

    def slots_of(self, s: int, t: np.ndarray) -> np.ndarray:
        """Physical slot of positions t of sequence s (the engine's page table)."""
        t = np.asarray(t, dtype=np.int64)
        return self.block_tables[s, t // BLOCK].astype(np.int64) * BLOCK + t % BLOCK

    def positions_call(self, pos_per_seq) -> WriteCall:
        rows, slots = [], []
        for s, t in enumerate(pos_per_seq):
            t = np.asarray(t, dtype=np.int64)
            rows.append(self.seq_start[s] + t)
            slots.append(self.slots_of(s, t))
        return WriteCall(np.concatenate(rows), np.concatenate(slots))


def make_workload(name, seed, num_seqs, num_q_heads, num_kv_heads, head_dim, kv, act,
                  lens=None, lens_range=None, num_blocks=None, planted=False, step_tokens=1,
                  prefill_chunk=0, chunks_per_call=16, partition_size=0) -> Workload:
    """Draw one workload. Either fixed `lens` or `lens_range` = (lo, hi) inclusive.

    The last `step_tokens` positions of each sequence form the timed step write; the rest
    is written by setup calls: one call, or `prefill_chunk`-token chunks (from position 0,
    never past the step), `chunks_per_call` chunks per call."""
    st_struct, st_q, st_k, st_v = np.random.SeedSequence(seed).spawn(4)
    rng = np.random.Generator(np.random.PCG64(st_struct))
    if lens is not None:
        L = np.asarray(lens, dtype=np.int32)
    else:
        L = rng.integers(lens_range[0], lens_range[1] + 1, size=num_seqs).astype(np.int32)
    nblk = -(-L.astype(np.int64) // BLOCK)
    used = int(nblk.sum())
    nb = used if num_blocks is None else int(num_blocks)
    assert nb >= used
    phys = rng.permutation(nb).astype(np.int32)
    mb = int(nblk.max())
    bt = np.full((num_seqs, mb), -1, dtype=np.int32)
    o = 0
    for s in range(num_seqs):
        bt[s, :nblk[s]] = phys[o:o + nblk[s]]
        o += nblk[s]
    pk = pv = None
    if planted:
        n = max(1, int(round(0.001 * num_kv_heads * head_dim)))
        pk = np.sort(rng.choice(num_kv_heads * head_dim, n, replace=False))
        pv = np.sort(rng.choice(num_kv_heads * head_dim, n, replace=False))
    q = _normal_rows(st_q, num_seqs, num_q_heads, head_dim, act)
    total = int(L.astype(np.int64).sum())
    k_rows = _normal_rows(st_k, total, num_kv_heads, head_dim, act, pk)
    v_rows = _normal_rows(st_v, total, num_kv_heads, head_dim, act, pv)
    start = np.concatenate([[0], np.cumsum(L.astype(np.int64))[:-1]])
    sm = float(np.float32(1.0) / np.sqrt(np.float32(head_dim)))
    w = Workload(name, seed, num_seqs, num_q_heads, num_kv_heads, head_dim, kv, act, L, nb, bt,
                 q, k_rows, v_rows, start, sm_scale=sm, partition_size=partition_size,
                 planted_k=pk, planted_v=pv)
    step_from = np.maximum(L.astype(np.int64) - step_tokens, 0)
    if prefill_chunk:
        chunks = []
        for s in range(num_seqs):
            for lo in range(0, int(step_from[s]), prefill_chunk):
                chunks.append((s, np.arange(lo, min(lo + prefill_chunk, int(step_from[s])))))
        for i in range(0, len(chunks), chunks_per_call):
            part = chunks[i:i + chunks_per_call]
            w.setup_calls.append(WriteCall(
                np.concatenate([w.seq_start[s] + t for s, t in part]),
                np.concatenate([w.slots_of(s, t) for s, t in part])))
    else:
        w.setup_calls.append(w.positions_call([np.arange(int(step_from[s])) for s in range(num_seqs)]))
    w.step_call = w.positions_call([np.arange(int(step_from[s]), int(L[s])) for s in range(num_seqs)])
    return w


def prefill_queries(w: Workload, n: int):
    """Multi-token queries for w: the last n_s = min(n, L_s) positions of every sequence.

    Returns (q bits [sum n_s, Hq, D] uint16, query_start [S + 1] int32). The rows are
    N(0, 1) in fp32 rounded to the activation dtype, drawn from the fifth child of the
    workload's root SeedSequence (the first four are structure, Q, K, V)."""
    ns = np.minimum(np.int64(n), w.context_lens.astype(np.int64))
    qs = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    st = np.random.SeedSequence(w.seed).spawn(5)[4]
    q = _normal_rows(st, int(qs[-1]), w.num_q_heads, w.head_dim, w.act)
    return q, qs


# The five workloads, full size. c1 is the tiny fp16 case; c2/c3 the 8B-shaped layer
# (32 q heads over 8 kv heads, head_dim 128, 64 sequences of 1k-8k tokens); c4 the 70B
# one-GPU tensor-parallel share (8 q heads over 1 kv head, 256 x 8192 tokens, FP8);
# c5 the same share at 64k-120k contexts with the 4-bit + fp16-outlier cache.
CONFIGS = {
    "c1": dict(seed=0, num_seqs=2, num_q_heads=4, num_kv_heads=1, head_dim=64, kv="f16",
               act="f16", lens=[37, 50], num_blocks=16),
    "c2": dict(seed=1, num_seqs=64, num_q_heads=32, num_kv_heads=8, head_dim=128, kv="bf16",
               act="bf16", lens_range=(1024, 8192), partition_size=768),
    "c3": dict(seed=2, num_seqs=64, num_q_heads=32, num_kv_heads=8, head_dim=128, kv="fp8",
               act="bf16", lens_range=(1024, 8192), planted=True, step_tokens=8,
               partition_size=768),
    "c4": dict(seed=3, num_seqs=256, num_q_heads=8, num_kv_heads=1, head_dim=128, kv="fp8",
               act="bf16", lens=[8192] * 256, planted=True, partition_size=0),
    "c5": dict(seed=4, num_seqs=32, num_q_heads=8, num_kv_heads=1, head_dim=128, kv="fp4",
               act="bf16", lens_range=(65536, 122880), planted=True, prefill_chunk=512,
               partition_size=512),
}

DESCRIPTIONS = {
    "c1": "tiny fp16: 2 seqs (37, 50 tokens), 4 q / 1 kv heads, D=64, 16-block pool",
    "c2": "8B-shaped bf16: 64 seqs x U[1k,8k], 32 q / 8 kv heads, D=128",
    "c3": "8B-shaped FP8 E4M3: 64 seqs x U[1k,8k], 32 q / 8 kv heads, D=128, 512-token write",
    "c4": "70B TP=8 one-GPU share FP8 E4M3: 256 seqs x 8192, 8 q / 1 kv head, D=128",
    "c5": "70B TP=8 one-GPU share FP4 E2M1 + fp16 outliers: 32 seqs x U[64k,120k], 8 q / 1 kv, D=128, split 512",
}


def config(name: str, **overrides) -> Workload:
    """A named workload; overrides shrink it for tests (e.g. num_seqs, lens, lens_range)."""
    kw = dict(CONFIGS[name])
    kw.update(overrides)
    if "lens" in overrides:
        kw.pop("lens_range", None)
    if "lens_range" in overrides:
        kw.pop("lens", None)
    if ("lens" in overrides or "lens_range" in overrides) and "num_blocks" not in overrides:
        kw.pop("num_blocks", None)
    return make_workload(name, **kw)
