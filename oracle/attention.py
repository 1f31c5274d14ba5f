"""Paged decode attention, exact, fp64 on the CPU.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg may import this package.

The decode path reaches, up to rounding order, a result with a plain definition: softmax
attention of each query head over the dequantized, gathered K/V of its sequence. This
module writes that definition out directly (no online softmax, no blocking):
  * gather through the block table (inferensys glossary "vLLM", PagedAttention entry);
  * the fused FP4 + fp16-outlier scores are exactly the scores of the dequantized cache
    (dailyaiworld.com, "Technical Breakdown: Dynamic Quantization with Outlier
    Retention", step 4: the fusion is lossless with respect to what is stored);
  * split-KV ("Flash-Decoding", same page and its cited sources): the context is cut into
    fixed partitions, each gives (o_p, lse_p), and the log-sum-exp merge recombines them.
Query head h reads kv head h // (Hq / Hkv) (grouped-query attention, contiguous groups).

Multi-token queries over the same cache (chunked prefill: a long prompt processed in
chunks, dailyaiworld.com, "vLLM 0.7 Ships Unified KV Cache Compression", engine diagram
with 512-token chunks, and inferensys glossary "vLLM", chunked prefill entry; draft
verification: the target model checks several proposed tokens at once, inferensys glossary
"vLLM", speculative decoding entry): the n queries of a sequence are its last n positions,
already written to the cache, and each attends causally to every position up to its own.
"""
from __future__ import annotations

import numpy as np

from .cache import Pool, gather_sequence
from .formats import act_decode


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float):
    """Exact softmax attention of one query q [D] over k, v [L, D] (fp64).

    Returns (out [D], lse) with z_t = sm_scale * q.k_t, out = sum_t softmax(z)_t v_t and
    lse = ln sum_t exp(z_t). L = 0 gives (zeros, -inf)."""
    if k.shape[0] == 0:
        return np.zeros(v.shape[1]), -np.inf
    z = sm_scale * (k @ q)
    m = z.max()
    p = np.exp(z - m)
    l = p.sum()
    return (p @ v) / l, m + np.log(l)


def decode_dense(q: np.ndarray, k_seq: np.ndarray, v_seq: np.ndarray, sm_scale: float,
                 partition_size: int = 0):
    """All query heads of one sequence. q [Hq, D]; k_seq, v_seq [L, Hkv, D].

    partition_size = 0: returns (out [Hq, D], lse [Hq]).
    partition_size > 0: returns per-partition (o [Hq, P, D], lse [Hq, P]) with partition p
    covering tokens [p*ps, min((p+1)*ps, L))."""
    hq = q.shape[0]
    hkv = k_seq.shape[1]
    assert hq % hkv == 0
    g = hq // hkv
    L = k_seq.shape[0]
    if partition_size == 0:
        out = np.zeros((hq, q.shape[1]))
        lse = np.zeros(hq)
        for h in range(hq):
            out[h], lse[h] = attend(q[h], k_seq[:, h // g, :], v_seq[:, h // g, :], sm_scale)
        return out, lse
    n_part = -(-L // partition_size)
    o = np.zeros((hq, n_part, q.shape[1]))
    lse = np.zeros((hq, n_part))
    for h in range(hq):
        for p in range(n_part):
            lo, hi = p * partition_size, min((p + 1) * partition_size, L)
            o[h, p], lse[h, p] = attend(q[h], k_seq[lo:hi, h // g, :], v_seq[lo:hi, h // g, :],
                                        sm_scale)
    return o, lse


def merge(o: np.ndarray, lse: np.ndarray):
    """Log-sum-exp merge of partitions. o [..., P, D], lse [..., P] -> (out [..., D],
    lse [...]). Partitions with lse = -inf get weight 0."""
    m = np.max(lse, axis=-1, keepdims=True)
    w = np.where(np.isneginf(lse), 0.0, np.exp(lse - m))
    tot = w.sum(axis=-1)
    out = (w[..., None] * o).sum(axis=-2) / tot[..., None]
    return out, m[..., 0] + np.log(tot)


def paged_decode(q_bits, act: str, pool: Pool, block_tables, context_lens, sm_scale: float,
                 k_scale=None, v_scale=None, partition_size: int = 0, seqs=None):
    """Decode for every sequence (or the listed ones) of a batch.

    q_bits [S, Hq, D] raw 16-bit bits. Returns dict seq -> (out, lse) or, with
    partition_size > 0, seq -> (o [Hq, P, D], lse [Hq, P])."""
    q = act_decode(q_bits, act)
    res = {}
    for s in (range(q.shape[0]) if seqs is None else seqs):
        k_seq, v_seq = gather_sequence(pool, block_tables[s], context_lens[s], k_scale, v_scale)
        res[s] = decode_dense(q[s], k_seq, v_seq, float(sm_scale), partition_size)
    return res


def paged_prefill(q_bits, act: str, pool: Pool, block_tables, context_lens, query_start,
                  sm_scale: float, k_scale=None, v_scale=None, seqs=None):
    """Multi-token queries for every sequence (or the listed ones) of a batch.

    q_bits [T, Hq, D] raw 16-bit bits, sequence s owning rows query_start[s] ..
    query_start[s + 1] - 1. With n = query_start[s + 1] - query_start[s] and L =
    context_lens[s], query i sits at position L - n + i and attends to positions
    0 .. L - n + i. Returns dict seq -> out [n, Hq, D]."""
    q = act_decode(q_bits, act)
    res = {}
    for s in (range(len(context_lens)) if seqs is None else seqs):
        L = int(context_lens[s])
        q0, q1 = int(query_start[s]), int(query_start[s + 1])
        n = q1 - q0
        k_seq, v_seq = gather_sequence(pool, block_tables[s], L, k_scale, v_scale)
        out = np.zeros((n, q.shape[1], q.shape[2]))
        for i in range(n):
            pos = L - n + i
            out[i], _ = decode_dense(q[q0 + i], k_seq[:pos + 1], v_seq[:pos + 1],
                                     float(sm_scale))
        res[s] = out
    return res
