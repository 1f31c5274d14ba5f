"""Pins of the oracle's paged decode attention and split-KV merge (CPU).

Pins: a pure-Python brute force over contiguous (unpaged) K/V on tiny inputs, torch's
scaled_dot_product_attention in float64 (a library routine the unpaged case reduces
to), bitwise invariance under relabelling of physical blocks, aliased block ids,
closed forms (one token, zero query, equal keys, two tokens), the fp16 pool equalling
unquantized attention, and the log-sum-exp identity merge(split) = unsplit."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import cache as C
from oracle import formats as F


def _brute(q, K, V, scale):
    """Softmax attention with Python floats and math.exp, one token at a time."""
    z = [scale * sum(qi * ki for qi, ki in zip(q, k)) for k in K]
    m = max(z)
    w = [math.exp(zi - m) for zi in z]
    tot = sum(w)
    out = [sum(w[t] * V[t][d] for t in range(len(V))) / tot for d in range(len(V[0]))]
    return out, m + math.log(tot)


def _f16_rows(rng, shape, scale=1.0):
    return F.f16_encode(rng.standard_normal(shape) * scale)


def _pool_with_sequences(rng, lens, hkv, d, nb, kind="f16"):
    """Write contiguous per-sequence rows into a shuffled f16 pool; returns the pool,
    block tables and the per-sequence rows."""
    pool = C.Pool.filled(kind, nb, hkv, d)
    phys = rng.permutation(nb)
    mb = max(-(-L // 16) for L in lens)
    bt = np.full((len(lens), mb), -1, dtype=np.int32)
    rows, used = [], 0
    for s, L in enumerate(lens):
        nblk = -(-L // 16)
        bt[s, :nblk] = phys[used:used + nblk]
        used += nblk
        k = _f16_rows(rng, (L, hkv, d))
        v = _f16_rows(rng, (L, hkv, d))
        t = np.arange(L)
        C.cache_write(pool, k, v, "f16", bt[s, t // 16].astype(np.int64) * 16 + t % 16)
        rows.append((k, v))
    return pool, bt, rows


def test_attend_matches_pure_python_brute_force():
    rng = np.random.default_rng(0)
    for L in (1, 2, 7, 33):
        q, K, V = rng.standard_normal(8), rng.standard_normal((L, 8)), rng.standard_normal((L, 8))
        out, lse = A.attend(q, K, V, 0.3)
        bo, bl = _brute(q.tolist(), K.tolist(), V.tolist(), 0.3)
        assert np.allclose(out, bo, rtol=1e-13, atol=1e-14)
        assert abs(lse - bl) < 1e-12


def test_attend_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(1)
    for L, d in ((5, 64), (300, 128), (4096, 128)):
        q, K, V = rng.standard_normal(d), rng.standard_normal((L, d)), rng.standard_normal((L, d))
        sc = 1 / math.sqrt(d)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, None, None], torch.from_numpy(K)[None, None],
            torch.from_numpy(V)[None, None], scale=sc)[0, 0, 0].numpy()
        out, _ = A.attend(q, K, V, sc)
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_paged_equals_dense_brute_force_with_gqa():
    rng = np.random.default_rng(2)
    lens, hkv, g, d = [37, 50, 16, 1], 2, 4, 64
    pool, bt, rows = _pool_with_sequences(rng, lens, hkv, d, nb=16)
    q_bits = _f16_rows(rng, (len(lens), hkv * g, d))
    res = A.paged_decode(q_bits, "f16", pool, bt, np.array(lens), 0.125)
    q = F.f16_decode(q_bits)
    for s, L in enumerate(lens):
        k, v = F.f16_decode(rows[s][0]), F.f16_decode(rows[s][1])
        for h in range(hkv * g):
            bo, bl = _brute(q[s, h].tolist(), k[:, h // g].tolist(), v[:, h // g].tolist(), 0.125)
            assert np.allclose(res[s][0][h], bo, rtol=1e-12, atol=1e-13)
            assert abs(res[s][1][h] - bl) < 1e-11


def test_block_relabelling_is_bitwise_invariant():
    rng = np.random.default_rng(3)
    lens, hkv, d, nb = [40, 70], 1, 64, 12
    pool, bt, _ = _pool_with_sequences(rng, lens, hkv, d, nb)
    q_bits = _f16_rows(rng, (2, 4, d))
    ref = A.paged_decode(q_bits, "f16", pool, bt, np.array(lens), 0.125)
    perm = rng.permutation(nb)  # new id of old block i is perm[i]
    pool2 = C.Pool.filled("f16", nb, hkv, d)
    for n in ("k", "v"):
        pool2.arrays[n][perm] = pool.arrays[n]
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1)
    got = A.paged_decode(q_bits, "f16", pool2, bt2, np.array(lens), 0.125)
    for s in range(2):
        assert np.array_equal(got[s][0], ref[s][0]) and np.array_equal(got[s][1], ref[s][1])


def test_aliased_block_ids_shared_prefix():
    rng = np.random.default_rng(4)
    pool, bt, rows = _pool_with_sequences(rng, [48], 1, 64, nb=6)
    # a second sequence shares the first two physical blocks, then has its own third
    bt2 = np.array([[bt[0, 0], bt[0, 1], bt[0, 2]], [bt[0, 0], bt[0, 1], 5]], dtype=np.int32)
    extra_k, extra_v = _f16_rows(rng, (16, 1, 64)), _f16_rows(rng, (16, 1, 64))
    C.cache_write(pool, extra_k, extra_v, "f16", 5 * 16 + np.arange(16))
    q_bits = _f16_rows(rng, (2, 4, 64))
    res = A.paged_decode(q_bits, "f16", pool, bt2, np.array([48, 40]), 0.125)
    q = F.f16_decode(q_bits)
    k1 = np.concatenate([F.f16_decode(rows[0][0])[:32], F.f16_decode(extra_k)[:8]])
    v1 = np.concatenate([F.f16_decode(rows[0][1])[:32], F.f16_decode(extra_v)[:8]])
    for h in range(4):
        o, _ = A.attend(q[1, h], k1[:, 0], v1[:, 0], 0.125)
        assert np.allclose(res[1][0][h], o, rtol=1e-13, atol=1e-14)


def test_closed_forms():
    rng = np.random.default_rng(5)
    V = rng.standard_normal((9, 16))
    K = rng.standard_normal((9, 16))
    # one token: the output is that token's value, lse = its logit
    o, lse = A.attend(rng.standard_normal(16), K[:1], V[:1], 0.25)
    assert np.array_equal(o, V[0])
    # zero query or equal keys: the output is the mean of V and lse = ln L (+ logit)
    o, lse = A.attend(np.zeros(16), K, V, 0.25)
    assert np.allclose(o, V.mean(axis=0), rtol=1e-14, atol=1e-15) and abs(lse - math.log(9)) < 1e-14
    q = rng.standard_normal(16)
    o, lse = A.attend(q, np.repeat(K[:1], 9, axis=0), V, 0.25)
    assert np.allclose(o, V.mean(axis=0), rtol=1e-14, atol=1e-15)
    assert abs(lse - (0.25 * q @ K[0] + math.log(9))) < 1e-13
    # two tokens with logit gap delta: weight of the first is 1 / (1 + e^-delta)
    k2 = np.zeros((2, 16))
    k2[0, 0], k2[1, 0] = 2.0, -1.0
    q2 = np.zeros(16)
    q2[0] = 1.0
    o, _ = A.attend(q2, k2, V[:2], 0.5)
    w = 1 / (1 + math.exp(-1.5))
    assert np.allclose(o, w * V[0] + (1 - w) * V[1], rtol=1e-14, atol=1e-15)


def test_f16_pool_equals_unquantized_attention():
    rng = np.random.default_rng(6)
    lens = [37, 50]
    pool, bt, rows = _pool_with_sequences(rng, lens, 1, 64, nb=16)
    q_bits = _f16_rows(rng, (2, 4, 64))
    res = A.paged_decode(q_bits, "f16", pool, bt, np.array(lens), 0.125)
    q = F.f16_decode(q_bits)
    for s in range(2):
        out, lse = A.decode_dense(q[s], F.f16_decode(rows[s][0]), F.f16_decode(rows[s][1]), 0.125)
        assert np.array_equal(res[s][0], out) and np.array_equal(res[s][1], lse)


@pytest.mark.parametrize("ps", [16, 32, 48, 512])
def test_merge_of_split_equals_unsplit(ps):
    rng = np.random.default_rng(7)
    q = rng.standard_normal((8, 128))
    k = rng.standard_normal((1000, 1, 128)) * 2
    v = rng.standard_normal((1000, 1, 128))
    out, lse = A.decode_dense(q, k, v, 1 / math.sqrt(128))
    o, l = A.decode_dense(q, k, v, 1 / math.sqrt(128), partition_size=ps)
    assert o.shape[1] == -(-1000 // ps)
    m, ml = A.merge(o, l)
    assert np.allclose(m, out, rtol=1e-12, atol=1e-13)
    assert np.allclose(ml, lse, rtol=1e-13, atol=1e-13)
    # one partition is the identity; an empty (-inf) partition has no weight
    m1, l1 = A.merge(out[:, None, :], lse[:, None])
    assert np.array_equal(m1, out) and np.array_equal(l1, lse)
    o_pad = np.concatenate([o, np.full((8, 1, 128), 123.0)], axis=1)
    l_pad = np.concatenate([l, np.full((8, 1), -np.inf)], axis=1)
    mp, lp = A.merge(o_pad, l_pad)
    assert np.allclose(mp, out, rtol=1e-12, atol=1e-13) and np.allclose(lp, lse, rtol=1e-13)


def _prefill_setup(seed, lens, ns, hq, hkv, d):
    rng = np.random.default_rng(seed)
    nb = sum(-(-L // 16) for L in lens) + 3
    pool, bt, rows = _pool_with_sequences(rng, lens, hkv, d, nb)
    qs = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    q = _f16_rows(rng, (int(qs[-1]), hq, d))
    return pool, bt, rows, qs, q


def test_prefill_single_query_is_decode():
    lens, ns, hq, hkv, d = [37, 50, 16], [1, 1, 1], 8, 2, 64
    pool, bt, rows, qs, q = _prefill_setup(1, lens, ns, hq, hkv, d)
    pre = A.paged_prefill(q, "f16", pool, bt, lens, qs, 0.125)
    dec = A.paged_decode(q, "f16", pool, bt, lens, 0.125)
    for s in range(len(lens)):
        assert np.array_equal(pre[s][0], dec[s][0])


def test_prefill_matches_masked_dense_brute_force():
    """Independent route: the whole causal score matrix of each sequence from its
    contiguous rows (no block table), masked with -inf, softmax over rows."""
    lens, ns, hq, hkv, d = [23, 40], [7, 17], 4, 1, 32
    pool, bt, rows, qs, q = _prefill_setup(2, lens, ns, hq, hkv, d)
    sc = 0.2
    pre = A.paged_prefill(q, "f16", pool, bt, lens, qs, sc)
    qv = F.f16_decode(q)
    for s, (L, n) in enumerate(zip(lens, ns)):
        k = F.f16_decode(rows[s][0])[:, 0, :]  # [L, D], one kv head
        v = F.f16_decode(rows[s][1])[:, 0, :]
        for h in range(hq):
            Q = qv[qs[s]:qs[s + 1], h, :]  # [n, D]
            z = sc * Q @ k.T  # [n, L]
            pos = L - n + np.arange(n)
            z = np.where(np.arange(L)[None, :] <= pos[:, None], z, -np.inf)
            w = np.exp(z - z.max(axis=1, keepdims=True))
            ref = (w @ v) / w.sum(axis=1, keepdims=True)
            assert np.allclose(pre[s][:, h, :], ref, rtol=1e-12, atol=1e-13)


def test_prefill_is_causal_and_ends_at_decode():
    """A query ignores cache positions after its own (they are overwritten with other
    values), and the chunk's last query equals decode over the whole context."""
    lens, ns, hq, hkv, d = [45], [12], 8, 2, 64
    pool, bt, rows, qs, q = _prefill_setup(3, lens, ns, hq, hkv, d)
    pre = A.paged_prefill(q, "f16", pool, bt, lens, qs, 0.125)
    L, n = lens[0], ns[0]
    rng = np.random.default_rng(9)
    t = np.arange(L - n + 5, L)  # positions after query 4 of the chunk
    junk = _f16_rows(rng, (len(t), hkv, d), scale=5.0)
    pool2 = C.Pool(pool.kind, pool.num_blocks, pool.num_kv_heads, pool.head_dim,
                   {k: a.copy() for k, a in pool.arrays.items()})
    C.cache_write(pool2, junk, junk, "f16", bt[0, t // 16].astype(np.int64) * 16 + t % 16)
    pre2 = A.paged_prefill(q, "f16", pool2, bt, lens, qs, 0.125)
    assert np.array_equal(pre[0][:5], pre2[0][:5])
    assert not np.allclose(pre[0][5:], pre2[0][5:])
    last = A.paged_decode(q[qs[1] - 1:qs[1]], "f16", pool, bt, lens, 0.125)
    assert np.array_equal(pre[0][n - 1], last[0][0])
