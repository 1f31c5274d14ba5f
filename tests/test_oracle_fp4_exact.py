"""Exact pins of the oracle's 4-bit path, from inputs whose encoding is known in advance.

The 4-bit scheme (dailyaiworld.com, "vLLM 0.7 Ships Unified KV Cache Compression",
"Technical Breakdown: Dynamic Quantization with Outlier Retention", steps 1-3) keeps the
channels whose norm reaches mean + 3.2 sigma in fp16 and stores every other value as an
E2M1 code times a per-token scale (largest inlier magnitude / 6). When every inlier of a
row is an E2M1 grid value times one power of two 2^k, with some inlier at +-6 * 2^k, the
scale is exactly 2^k, every code is the grid index itself and dequantization must give the
input back bit for bit; an outlier value that fp16 holds exactly must come back exactly
too. Each token and each of K and V gets its own power of two, so a scale read from the
wrong token offset, or K's scale used for V, changes the result by a factor of two or
more. The rows land in the block over several calls, in scrambled order.

The second test builds a block whose candidate channel sits within 1e-5 (relative) of the
threshold, the case where fp32 statistics on the GPU and fp64 ones in the oracle may
disagree, and checks that the replay counts it and that the pool comparison masks it (and
only it)."""
import os
import sys

import numpy as np
import pytest

from oracle import cache as C
from oracle.formats import act_decode

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from oracle_side import NEAR_TIE, assert_pool_equal  # noqa: E402

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])  # E2M1 magnitudes, code order


def _bits(x, act):
    """Values that the activation dtype holds exactly -> raw 16-bit patterns."""
    x = np.asarray(x, dtype=np.float32)
    if act == "f16":
        b = x.astype(np.float16)
        assert np.array_equal(b.astype(np.float32), x)
        return b.view(np.uint16)
    u = x.view(np.uint32)
    assert np.all(u & 0xFFFF == 0), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def _exact_rows(rng, n, d, exps, outlier_ch):
    """Rows [n, d] of grid values times 2^exps[t], each with an inlier at +-6 * 2^e, and
    channel outlier_ch at +-64 * 2^e (exact in fp16 and bf16). Returns the values, the code
    each inlier must get (sign bit | grid index) and the per-token scales 2^e."""
    idx = rng.integers(0, 8, (n, d))
    sign = rng.integers(0, 2, (n, d))
    for t in range(n):
        c = (outlier_ch + 1 + rng.integers(0, d - 1)) % d  # some inlier channel holds +-6
        idx[t, c] = 7
    scale = np.ldexp(1.0, np.asarray(exps))
    x = np.where(sign == 1, -1.0, 1.0) * GRID[idx] * scale[:, None]
    x[:, outlier_ch] = np.where(sign[:, outlier_ch] == 1, -64.0, 64.0) * scale
    codes = (idx | (sign << 3)).astype(np.uint8)
    codes[:, outlier_ch] = 0  # code +0 at an outlier channel
    return x, codes, scale


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
def test_fp4_dequant_exact_on_power_of_two_rows(d, act):
    rng = np.random.default_rng(100 + d)
    nb, hkv = 3, 2
    blk = 1  # the block under test; blocks 0 and 2 hold other tokens
    out_k, out_v = 5, d - 3  # one outlier channel per side, different for K and V
    k_exp = np.arange(16) - 7          # token t of K: 2^(t - 7) (outliers stay in fp16 range)
    v_exp = 5 - (np.arange(16) * 7) % 12  # V: another power of two per token
    kx, kcodes, ks = _exact_rows(rng, 16, d, k_exp, out_k)
    vx, vcodes, vs = _exact_rows(rng, 16, d, v_exp, out_v)
    # head 1 gets the same rows scaled by 2 (a wrong head offset changes every value)
    k_rows = np.stack([kx, 2.0 * kx], 1)
    v_rows = np.stack([vx, 2.0 * vx], 1)
    kb, vb = _bits(k_rows, act), _bits(v_rows, act)

    pool = C.Pool.filled("fp4", nb, hkv, d)
    order = rng.permutation(16)
    # three calls: the first opens the block (5 tokens decide its outlier set), the other
    # two reuse it; each call also writes a row into another block
    for part in (order[:5], order[5:11], order[11:]):
        slots = np.concatenate([blk * 16 + part, [0 * 16 + int(part[0]), 2 * 16 + int(part[-1])]])
        krow = np.concatenate([kb[part], kb[part[:1]], kb[part[-1:]]])
        vrow = np.concatenate([vb[part], vb[part[:1]], vb[part[-1:]]])
        C.cache_write(pool, krow, vrow, act, slots.astype(np.int64))

    t = np.arange(16)
    k_hat, v_hat = C.dequant_slot_rows(pool, np.full(16, blk), t)
    for got, want in ((k_hat, k_rows), (v_hat, v_rows)):
        assert got.dtype == np.float64
        assert np.array_equal(got, want)  # exact: inliers, scales and outliers
    for name, codes, sc, och in (("k", kcodes, ks, out_k), ("v", vcodes, vs, out_v)):
        rec = C.fp4_records(pool, name)[blk]
        for h in range(hkv):
            assert rec[h, 0] == 1 and rec[h, 1] == och and np.all(rec[h, 2:] == 0xFF)
            assert np.array_equal(C.fp4_scales(pool, name)[blk, h].astype(np.float64),
                                  sc * (1.0, 2.0)[h])
            assert np.array_equal(C.fp4_get_codes(pool, name)[blk, h], codes)


def _near_tie_rows(d, act):
    """One block of 16 rows [16, d] whose channel 0 norm is within 1e-5 of the threshold."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((16, d)).astype(np.float32)
    x = act_decode(_bits_round(x, act), act)
    # channel 0: tokens 2..15 at a, tokens 0 and 1 at u and v; pick (a, u, v) among the
    # dtype's values so that r_0 - (mu + 3.2 sigma) is closest to 0
    r_other = np.sqrt(np.mean(x[:, 1:] ** 2, axis=0))

    def margin(r0):
        r = np.concatenate([[r0], r_other])
        thr = r.mean() + 3.2 * r.std()
        return (r0 - thr) / thr

    lo, hi = 0.0, 50.0
    for _ in range(200):  # margin(r0) increases with r0 here
        mid = (lo + hi) / 2
        lo, hi = (mid, hi) if margin(mid) < 0 else (lo, mid)
    target = (lo + hi) / 2
    step = np.spacing(np.float16(target)) if act == "f16" else 2.0 ** (np.floor(np.log2(target)) - 7)
    a = float(act_decode(_bits_round(np.float32(target), act), act))
    cand = a + step * np.arange(-40, 41)
    u, v = np.meshgrid(cand, cand, indexing="ij")
    r0 = np.sqrt((u ** 2 + v ** 2 + 14 * a * a) / 16)
    mu = (r0 + r_other.sum()) / d
    var = ((r0 - mu) ** 2 + ((r_other[None, None, :] - mu[..., None]) ** 2).sum(-1)) / d
    thr = mu + 3.2 * np.sqrt(var)
    m = np.abs(r0 - thr) / thr
    i, j = np.unravel_index(np.argmin(m), m.shape)
    x[:, 0] = a
    x[0, 0], x[1, 0] = u[i, j], v[i, j]
    return x


def _bits_round(x, act):
    x = np.asarray(x, dtype=np.float32)
    if act == "f16":
        return x.astype(np.float16).view(np.uint16)
    u = np.atleast_1d(x).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16).reshape(np.shape(x))


@pytest.mark.parametrize("act", ["bf16", "f16"])
def test_near_tie_is_counted_and_masked(act):
    d, nb = 128, 2
    x = _near_tie_rows(d, act)
    assert C.fp4_calibration_margin(x) <= NEAR_TIE  # the construction reached a near-tie
    rng = np.random.default_rng(8)
    far = rng.standard_normal((16, d)).astype(np.float32)
    far[:, 9] *= 20.0  # block 1: a clear outlier, far from any tie
    k_rows = np.stack([_bits_round(x, act), _bits_round(far, act)])  # [blocks, 16, d]
    k_rows = k_rows.reshape(32, 1, d)
    v_rows = _bits_round(np.ones((32, 1, d), dtype=np.float32), act)  # sigma = 0: no tie
    pool = C.Pool.filled("fp4", nb, 1, d)
    log = []
    C.cache_write(pool, k_rows, v_rows, act, np.arange(32, dtype=np.int64), calib_log=log)
    near = {(n, b, h) for (n, b, h, m) in log if m <= NEAR_TIE}
    assert near == {("k", 0, 0)}  # counted, and only it
    assert len(log) == 4  # K and V of both blocks were calibrated

    # a device pool that differs from the oracle's only in the near-tie tile passes with
    # the mask and fails without it; a difference elsewhere fails either way
    dev = {n: a.copy().reshape(-1).view(np.uint8) for n, a in pool.arrays.items()}
    dev["k"].reshape(nb, 1, -1)[0, 0, 3] ^= 0x11
    assert_pool_equal(dev, pool, near=near)
    with pytest.raises(AssertionError):
        assert_pool_equal(dev, pool)
    dev["k"].reshape(nb, 1, -1)[1, 0, 3] ^= 0x11
    with pytest.raises(AssertionError):
        assert_pool_equal(dev, pool, near=near)
