"""GPU parity of whole-block copies (pa_copy_blocks) and of copy on write driven by the
host block allocator, against the oracle's copy (oracle/blocks.py) on the same inputs.

Pools must match the oracle byte for byte after every copy (destinations, untouched
blocks and sentinels alike), in every format: copies inside one pool, swaps out to a pool
in pinned host memory and back in, pair lists in device or pinned host memory, pairs with
out-of-range ids (skipped and flagged), and a full-size pool. Decode over the moved
blocks stays within max-abs 2e-3 and relative L2 1e-2 of the oracle's exact attention."""
import numpy as np
import pytest

from oracle import blocks as OB
from oracle import cache as C
from oracle_side import assert_close, assert_pool_equal, oracle_decode, replay
from workload import config

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from test_parity_gpu import _say  # noqa: E402

# format -> (workload, overrides): small shapes with ragged tails and spare blocks
CASES = {
    "f16": ("c1", dict(num_blocks=24)),
    "bf16": ("c2", dict(num_seqs=3, lens=[300, 77, 16], num_blocks=48)),
    "fp8": ("c4", dict(num_seqs=3, lens=[300, 77, 16], num_blocks=48)),
    "bf8": ("c4", dict(num_seqs=3, lens=[300, 77, 16], num_blocks=48, kv="bf8")),
    "fp8t": ("c3", dict(num_seqs=3, lens=[300, 77, 16], num_blocks=48, kv="fp8t")),
    "bf8t": ("c4", dict(num_seqs=3, lens=[300, 77, 16], num_blocks=48, kv="bf8t")),
    "fp4": ("c5", dict(num_seqs=3, lens=[300, 77, 16], num_blocks=48)),
}


def _prepared(kind):
    from paged_quantized_kv_reshape_amd.harness import DeviceRun
    base, over = CASES[kind]
    w = config(base, **over)
    assert w.kv == kind
    run = DeviceRun(w, partition_size=0)
    run.prepare()
    torch.cuda.synchronize()
    pool, ks, vs, near = replay(w)
    assert len(near) == 0
    return w, run, pool, ks, vs


def _pairs(p, where="cuda"):
    t = torch.from_numpy(np.asarray(p, dtype=np.int32).reshape(-1, 2).copy())
    return t.cuda() if where == "cuda" else t.pin_memory()


def _free_ids(w):
    used = set(w.block_tables[w.block_tables >= 0].tolist())
    return [b for b in range(w.num_blocks) if b not in used]


def _decode_check(w, run, pool, ks, vs, what):
    run.decode()
    torch.cuda.synchronize()
    assert run.device_error() == 0
    ref = oracle_decode(w, pool, ks, vs, range(w.num_seqs))
    assert_close(run.out.cpu().numpy(), np.stack([ref[s][0] for s in range(w.num_seqs)]), what)


@pytest.mark.parametrize("kind", list(CASES))
def test_copy_within_pool(kind):
    """Copy on write: sequence 0's blocks duplicated into free blocks, its table pointed at
    the copies; pool bytes and decode against the oracle."""
    from paged_quantized_kv_reshape_amd import pa_copy_blocks
    w, run, pool, ks, vs = _prepared(kind)
    n0 = -(-int(w.context_lens[0]) // 16)
    free = _free_ids(w)[:n0]
    pairs = np.stack([w.block_tables[0, :n0], free], 1)
    _say(f"[copy] {kind}: {n0} blocks of seq 0 -> {free[:4]}...")
    pa_copy_blocks(run.pool, run.pool, _pairs(pairs), run.dev_err)
    OB.copy_blocks(pool, pool, pairs)
    torch.cuda.synchronize()
    assert run.device_error() == 0
    assert_pool_equal(run.pool.numpy(), pool)
    w.block_tables[0, :n0] = free
    run.block_tables[0, :n0] = torch.tensor(free, dtype=torch.int32, device="cuda")
    _decode_check(w, run, pool, ks, vs, f"{kind} after copy")


@pytest.mark.parametrize("pairs_where", ["cuda", "pinned"])
@pytest.mark.parametrize("kind", list(CASES))
def test_swap_out_and_back_in(kind, pairs_where):
    """Sequence 1's blocks swapped out to a pinned host pool, the device blocks scrambled
    (reused by another sequence meanwhile), then swapped back in to other ids."""
    from paged_quantized_kv_reshape_amd import KVPool, pa_copy_blocks
    w, run, pool, ks, vs = _prepared(kind)
    n1 = -(-int(w.context_lens[1]) // 16)
    nbh = n1 + 5
    host = KVPool(kind, nbh, w.num_kv_heads, w.head_dim, device="cpu", fill=0x3C)
    ohost = C.Pool.filled(kind, nbh, w.num_kv_heads, w.head_dim, sentinel=0x3C)
    out_ids = list(range(nbh - 1, nbh - 1 - n1, -1))
    src = w.block_tables[1, :n1].copy()
    pairs = np.stack([src, out_ids], 1)
    _say(f"[swap] {kind} pairs in {pairs_where}: {n1} blocks out")
    pa_copy_blocks(run.pool, host, _pairs(pairs, pairs_where), run.dev_err)
    OB.copy_blocks(pool, ohost, pairs)
    torch.cuda.synchronize()
    assert run.device_error() == 0
    assert_pool_equal(host.numpy(), ohost)
    # another sequence overwrites the swapped-out blocks (torch fill, on both sides)
    idx = torch.from_numpy(src.astype(np.int64)).cuda()
    for name, t in run.pool.bytes.items():
        t.view(w.num_blocks, -1).index_fill_(0, idx, 0x11)
        pool.arrays[name].view(np.uint8).reshape(w.num_blocks, -1)[src] = 0x11
    # back in, into the free blocks
    new_ids = _free_ids(w)[:n1]
    back = np.stack([out_ids, new_ids], 1)
    pa_copy_blocks(host, run.pool, _pairs(back, pairs_where), run.dev_err)
    OB.copy_blocks(ohost, pool, back)
    torch.cuda.synchronize()
    assert run.device_error() == 0
    assert_pool_equal(run.pool.numpy(), pool)
    w.block_tables[1, :n1] = new_ids
    run.block_tables[1, :n1] = torch.tensor(new_ids, dtype=torch.int32, device="cuda")
    _decode_check(w, run, pool, ks, vs, f"{kind} after swap")


def test_out_of_range_pairs_are_skipped_and_flagged():
    from paged_quantized_kv_reshape_amd import KVPool, pa_copy_blocks
    w, run, pool, ks, vs = _prepared("fp4")
    host = KVPool("fp4", 6, w.num_kv_heads, w.head_dim, device="cpu", fill=0x3C)
    ohost = C.Pool.filled("fp4", 6, w.num_kv_heads, w.head_dim, sentinel=0x3C)
    good = [[int(w.block_tables[0, 0]), 0], [int(w.block_tables[0, 1]), 5]]
    bad = [[-1, 1], [w.num_blocks, 2], [int(w.block_tables[0, 2]), 6], [3, -7]]
    p = good[:1] + bad[:2] + good[1:] + bad[2:]
    pa_copy_blocks(run.pool, host, _pairs(p), run.dev_err)
    OB.copy_blocks(pool, ohost, good)
    torch.cuda.synchronize()
    assert run.device_error() == 1  # PA_DEVERR_BAD_BLOCK
    assert_pool_equal(host.numpy(), ohost)


def test_full_size_pool_copy_and_swap():
    """The 70B one-GPU share's FP8 pool (32768 blocks of 2 KB per side) filled with
    seeded random bytes: 16384 copies inside the pool, then 4096 blocks out to a pinned
    host pool and back, against the same copies done by the oracle."""
    from paged_quantized_kv_reshape_amd import KVPool, pa_copy_blocks
    nb, hkv, d = 32768, 1, 128
    rng = np.random.default_rng(21)
    ones = torch.ones(hkv, dtype=torch.float32, device="cuda")
    dev = KVPool("fp8", nb, hkv, d, k_scale=ones, v_scale=ones)
    opool = C.Pool.filled("fp8", nb, hkv, d)
    for name, a in opool.arrays.items():
        a[...] = rng.integers(0, 256, size=a.shape, dtype=np.uint8)
        dev.bytes[name].copy_(torch.from_numpy(a.reshape(-1)))
    perm = rng.permutation(nb)
    pairs = np.stack([perm[:16384], perm[16384:]], 1)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    _say("[full] 16384 in-pool copies")
    pa_copy_blocks(dev, dev, _pairs(pairs), err)
    OB.copy_blocks(opool, opool, pairs)
    host = KVPool("fp8", 4096, hkv, d, device="cpu", fill=0)
    ohost = C.Pool.filled("fp8", 4096, hkv, d, sentinel=0)
    out = np.stack([rng.choice(nb, 4096, replace=False), rng.permutation(4096)], 1)
    _say("[full] 4096 blocks out to host")
    pa_copy_blocks(dev, host, _pairs(out), err)
    OB.copy_blocks(opool, ohost, out)
    back = np.stack([np.arange(4096), rng.choice(nb, 4096, replace=False)], 1)
    _say("[full] 4096 blocks back in")
    pa_copy_blocks(host, dev, _pairs(back, "pinned"), err)
    OB.copy_blocks(ohost, opool, back)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert_pool_equal(host.numpy(), ohost)
    assert_pool_equal(dev.numpy(), opool)


def _bits(x, act):
    x = np.asarray(x, dtype=np.float32)
    if act == "f16":
        return x.astype(np.float16).view(np.uint16)
    u = x.view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("kind", ["fp8", "fp8t", "fp4", "bf16"])
def test_beam_fork_copy_on_write(kind):
    """A sequence of 41 tokens forks into two beams that share its 3 blocks (the last one
    partial). Each beam then appends 30 tokens of its own: the allocator's copy on write
    gives the first writer a copy of the shared partial block (pa_copy_blocks), the second
    writes in place, and both spill into fresh blocks. Pools and both beams' decode
    against the oracle doing the same steps."""
    from paged_quantized_kv_reshape_amd import (BlockAllocator, KVPool, pa_cache_write,
                                                pa_copy_blocks, pa_decode)
    hkv, hq, d, nb = 2, 8, 128, 16
    act = "bf16"
    rng = np.random.default_rng(31)
    x = rng.standard_normal((2, 41 + 60, hkv, d)).astype(np.float32)
    x[:, :, :, 9] *= 20.0
    kb, vb = _bits(x[0], act), _bits(x[1], act)
    ks = vs = None
    dks = dvs = None
    if kind == "fp8":
        ks, vs = C.fp8_head_scale(kb, act, "e4m3"), C.fp8_head_scale(vb, act, "e4m3")
        dks, dvs = torch.from_numpy(ks).cuda(), torch.from_numpy(vs).cuda()
    dev = KVPool(kind, nb, hkv, d, fill=0xA5, k_scale=dks, v_scale=dvs)
    opool = C.Pool.filled(kind, nb, hkv, d)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    alloc = BlockAllocator(nb)

    def write(rows, slots):
        slots = np.asarray(slots, dtype=np.int64)
        C.cache_write(opool, kb[rows], vb[rows], act, slots, ks, vs)
        kt = torch.from_numpy(kb[rows].view(np.int16)).cuda().view(torch.bfloat16)
        vt = torch.from_numpy(vb[rows].view(np.int16)).cuda().view(torch.bfloat16)
        pa_cache_write(dev, kt, vt, torch.from_numpy(slots).cuda(), err)

    # prefill of the shared prefix
    table_a = alloc.alloc(3)
    write(np.arange(41), [table_a[t // 16] * 16 + t % 16 for t in range(41)])
    alloc.share(table_a)
    table_b = list(table_a)
    assert alloc.refcount(table_a[2]) == 2
    # each beam appends 30 tokens (rows 41..70 for A, 71..100 for B)
    for beam, (table, first_row) in enumerate(((table_a, 41), (table_b, 71))):
        last = table[-1]
        new, copy = alloc.writable(last)
        assert copy == (beam == 0)  # the second writer finds the block its own
        if copy:
            pa_copy_blocks(dev, dev, _pairs([[last, new]]), err)
            OB.copy_blocks(opool, opool, [[last, new]])
            table[-1] = new
        table += alloc.alloc(2)  # positions 48..79 spill into two fresh blocks
        pos = np.arange(41, 71)
        write(first_row + np.arange(30), [table[p // 16] * 16 + p % 16 for p in pos])
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert alloc.refcount(table_a[0]) == 2 and alloc.refcount(table_a[2]) == 1
    assert_pool_equal(dev.numpy(), opool)
    q = _bits(rng.standard_normal((2, hq, d)), act)
    bt = np.array([table_a, table_b], dtype=np.int32)
    cl = np.array([71, 71], dtype=np.int32)
    out = torch.empty((2, hq, d), dtype=torch.float32, device="cuda")
    pa_decode(torch.from_numpy(q.view(np.int16)).cuda().view(torch.bfloat16), dev,
              torch.from_numpy(bt).cuda(), torch.from_numpy(cl).cuda(), 1.0 / np.sqrt(d), 0,
              out, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    from oracle import attention as A
    ref = A.paged_decode(q, act, opool, bt, cl, 1.0 / np.sqrt(d), ks, vs)
    assert_close(out.cpu().numpy(), np.stack([ref[0][0], ref[1][0]]), f"{kind} beams")
    # the beams differ only after the fork
    assert not np.allclose(ref[0][0], ref[1][0])
    # beams finish: every block goes back, freed FP4 blocks are re-armed
    freed = alloc.release(table_a) + alloc.release(table_b)
    assert sorted(freed) == sorted(set(table_a) | set(table_b)) and alloc.num_free == nb
    alloc.close()
