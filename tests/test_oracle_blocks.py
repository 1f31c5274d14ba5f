"""Pins of the oracle's whole-block copy (oracle/blocks.py) to what a copy must preserve.

A copied block must be indistinguishable from its source to every later reader: decode of
a sequence whose table names the copies equals decode over the originals, bit for bit, in
every pool format (FP4 blocks here hold two outliers, so the second one lives in the
outlier slot array, which a copy must move too); a swap out to another pool and back into
new ids restores every byte; blocks that no pair names keep theirs. A copy that forgets
one of the pool's arrays is shown to fail the decode pin."""
import numpy as np
import pytest

from oracle import attention as A
from oracle import blocks as B
from oracle import cache as C

D, HKV, HQ = 128, 2, 4


def _bits(x, act):
    x = np.asarray(x, dtype=np.float32)
    if act == "f16":
        return x.astype(np.float16).view(np.uint16)
    u = x.view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _written_pool(kind, nb, lens, seed=0):
    """A pool of nb blocks holding sequences of the given lengths, written token by token
    in one call per sequence, block ids shuffled; returns (pool, tables, scales)."""
    rng = np.random.default_rng(seed)
    act = "f16" if kind == "f16" else "bf16"
    ids = rng.permutation(nb)
    nblk = [-(-L // 16) for L in lens]
    tables = np.full((len(lens), max(nblk)), -1, dtype=np.int32)
    pos = 0
    for s, n in enumerate(nblk):
        tables[s, :n] = ids[pos:pos + n]
        pos += n
    pool = C.Pool.filled(kind, nb, HKV, D)
    T = sum(lens)
    x = rng.standard_normal((2, T, HKV, D)).astype(np.float32)
    x[:, :, :, [5, 77]] *= 20.0  # two outlier channels per (block, head)
    kb, vb = _bits(x[0], act), _bits(x[1], act)
    ks = vs = None
    if kind in ("fp8", "bf8"):
        fmt = C.FP8_KINDS[kind][0]
        ks, vs = C.fp8_head_scale(kb, act, fmt), C.fp8_head_scale(vb, act, fmt)
    start = 0
    for s, L in enumerate(lens):
        t = np.arange(L)
        slots = tables[s, t // 16].astype(np.int64) * 16 + t % 16
        C.cache_write(pool, kb[start:start + L], vb[start:start + L], act, slots, ks, vs)
        start += L
    return pool, tables, (ks, vs, act)


def _decode(pool, tables, lens, sc, seed=1):
    ks, vs, act = sc
    rng = np.random.default_rng(seed)
    q = _bits(rng.standard_normal((len(lens), HQ, D)), act)
    res = A.paged_decode(q, act, pool, tables, np.asarray(lens, dtype=np.int32),
                         1.0 / np.sqrt(D), ks, vs)
    return np.stack([res[s][0] for s in range(len(lens))])


KINDS = ["f16", "fp8", "bf8", "fp8t", "fp4"]


@pytest.mark.parametrize("kind", KINDS)
def test_copy_within_pool_preserves_decode(kind):
    lens = [70, 33]
    pool, tables, sc = _written_pool(kind, 24, lens)
    if kind == "fp4":
        cnt = C.fp4_records(pool, "k")[tables[0, :4], :, 0]
        assert (cnt == 2).all()  # the second outlier sits in the slot array
    want = _decode(pool, tables, lens, sc)
    used = set(tables[tables >= 0].tolist())
    free = [b for b in range(24) if b not in used]
    n0 = -(-lens[0] // 16)
    pairs = np.stack([tables[0, :n0], free[:n0]], 1)
    before = {k: a.copy() for k, a in pool.arrays.items()}
    B.copy_blocks(pool, pool, pairs)
    t2 = tables.copy()
    t2[0, :n0] = free[:n0]
    got = _decode(pool, t2, lens, sc)
    assert np.array_equal(got, want)
    # blocks that no pair names keep every byte
    keep = [b for b in range(24) if b not in set(free[:n0])]
    for k, a in pool.arrays.items():
        assert np.array_equal(a[keep], before[k][keep])


@pytest.mark.parametrize("kind", KINDS)
def test_swap_out_and_back_restores_bytes_and_decode(kind):
    lens = [50, 64, 17]
    pool, tables, sc = _written_pool(kind, 16, lens, seed=3)
    want = _decode(pool, tables, lens, sc)
    host = C.Pool.filled(kind, 9, HKV, D, sentinel=0x3C)
    n1 = -(-lens[1] // 16)
    out_ids = np.arange(9)[::-1][:n1]
    B.copy_blocks(pool, host, np.stack([tables[1, :n1], out_ids], 1))
    snapshot = {k: a[tables[1, :n1]].copy() for k, a in pool.arrays.items()}
    # the device blocks are reused by someone else meanwhile
    for k, a in pool.arrays.items():
        a[tables[1, :n1]] = 0x11
    # swap back in, into other ids: the sequence's former blocks 1..n1 rotate by one
    new_ids = np.roll(tables[1, :n1], 1)
    B.copy_blocks(host, pool, np.stack([out_ids, new_ids], 1))
    for k, a in pool.arrays.items():
        assert np.array_equal(a[new_ids], snapshot[k])
    t2 = tables.copy()
    t2[1, :n1] = new_ids
    assert np.array_equal(_decode(pool, t2, lens, sc), want)


def test_a_copy_that_skips_an_array_fails_the_decode_pin():
    """The decode pin sees the FP4 outlier slot array: leaving it behind changes decode."""
    lens = [48]
    pool, tables, sc = _written_pool("fp4", 8, lens, seed=5)
    want = _decode(pool, tables, lens, sc)
    n = 3
    free = [b for b in range(8) if b not in set(tables[0, :n].tolist())][:n]
    for name, arr in pool.arrays.items():  # the planted mistake: out_val arrays stay put
        if "out_val" not in name:
            arr[free] = arr[tables[0, :n]]
    t2 = tables.copy()
    t2[0, :n] = free
    assert not np.array_equal(_decode(pool, t2, lens, sc), want)


def test_copy_preconditions():
    p = C.Pool.filled("fp8", 8, HKV, D)
    with pytest.raises(AssertionError):
        B.copy_blocks(p, p, [[0, 1], [2, 1]])  # duplicate destination
    with pytest.raises(AssertionError):
        B.copy_blocks(p, p, [[0, 1], [1, 2]])  # destination 1 is also a source
    with pytest.raises(AssertionError):
        B.copy_blocks(p, C.Pool.filled("bf8", 8, HKV, D), [[0, 1]])  # other format
    with pytest.raises(AssertionError):
        B.copy_blocks(p, p, [[0, 8]])  # outside the pool
    B.copy_blocks(p, p, np.zeros((0, 2), dtype=np.int64))  # nothing to do
