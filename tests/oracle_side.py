"""Oracle-side replay of a workload and the parity checks (test infrastructure)."""
import numpy as np

from oracle import attention as A
from oracle import cache as C

# Decode tolerance: elementwise max |gpu - oracle| <= 2e-3 and relative L2 error <= 1e-2,
# in fp32, against exact attention on the identical dequantized cache.
ATOL = 2e-3
RTOL_L2 = 1e-2
# FP4 outlier sets are decided by fp32 statistics on the GPU and fp64 ones in the oracle;
# a (block, head) whose closest channel sits within this relative distance of the
# threshold is a near-tie and is excluded from the bit-exact comparison (and counted).
NEAR_TIE = 1e-5


def replay(w, only_blocks=None):
    """Oracle pool after every write call of the workload (setup, then step)."""
    pool = C.Pool.filled(w.kv, w.num_blocks, w.num_kv_heads, w.head_dim)
    ks = vs = None
    if w.kv in ("fp8", "bf8"):
        fmt = C.FP8_KINDS[w.kv][0]
        ks = C.fp8_head_scale(w.k_rows, w.act, fmt)
        vs = C.fp8_head_scale(w.v_rows, w.act, fmt)
    log = []
    keep = None if only_blocks is None else np.asarray(sorted(only_blocks))
    for call in list(w.setup_calls) + [w.step_call]:
        rows, slots = call.rows, call.slots
        if keep is not None:
            sel = np.isin(slots // 16, keep)
            rows, slots = rows[sel], slots[sel]
            if len(rows) == 0:
                continue
        C.cache_write(pool, w.k_rows[rows], w.v_rows[rows], w.act, slots, ks, vs,
                      calib_log=log)
    near = {(n, b, h) for (n, b, h, m) in log if m <= NEAR_TIE}
    return pool, ks, vs, near


def seq_blocks(w, seqs):
    out = set()
    for s in seqs:
        n = -(-int(w.context_lens[s]) // 16)
        out.update(int(b) for b in w.block_tables[s, :n])
    return out


def assert_pool_equal(gpu_bytes, opool, blocks=None, near=()):
    """Bit-exact comparison of every pool array (optionally only some physical blocks).
    FP4 (block, head) near-ties are masked out of K or V arrays, per side."""
    for name, arr in opool.arrays.items():
        g = gpu_bytes[name].view(arr.dtype).reshape(arr.shape)
        o = arr
        if blocks is not None:
            idx = np.asarray(sorted(blocks))
            g, o = g[idx], o[idx]
            bmap = {b: i for i, b in enumerate(idx)}
        else:
            bmap = None
        side = name[0]
        ok = np.ones(o.shape[:2], dtype=bool)
        for (n, b, h) in near:
            if n == side:
                bi = bmap.get(b) if bmap is not None else b
                if bi is not None:
                    ok[bi, h] = False
        gb = g.view(np.uint8).reshape(o.shape[0], o.shape[1], -1)
        ob = o.view(np.uint8).reshape(o.shape[0], o.shape[1], -1)
        bad = np.nonzero((gb != ob).any(axis=2) & ok)
        if len(bad[0]):
            b, h = int(bad[0][0]), int(bad[1][0])
            raise AssertionError(
                f"{name}: {len(bad[0])} (block, head) tiles differ; first at block index {b}, "
                f"head {h}: gpu {gb[b, h][:24].tolist()} oracle {ob[b, h][:24].tolist()}")


def assert_close(got, want, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - want)
    rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
    assert err.max() <= ATOL, f"{what}: max abs err {err.max():.3e} > {ATOL} (rel L2 {rel:.2e})"
    assert rel <= RTOL_L2, f"{what}: rel L2 err {rel:.3e} > {RTOL_L2}"
    return float(err.max()), float(rel)


def oracle_decode(w, pool, ks, vs, seqs, partition_size=0):
    return A.paged_decode(w.q, w.act, pool, w.block_tables, w.context_lens, w.sm_scale, ks, vs,
                          partition_size=partition_size, seqs=seqs)
