"""Pins of the oracle's cache write, FP4 outlier calibration and dequantization (CPU).

Closed forms and invariants the pages and the mathematics fix: slot placement with
sentinel bytes, the k-equal-channels threshold closed form (which also shows the outlier
capacity is tight), the planted x20 channel, sigma = 0, per-token scale and per-head
scale invariants (the absmax element lands on the largest code), and dequantization
error bounds."""
import numpy as np
import pytest

from oracle import cache as C
from oracle import formats as F


def _bf16_bits(x):
    """fp32 -> bf16 bits, round to nearest even (test-side input preparation)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def test_outlier_capacity_closed_form():
    assert C.outlier_capacity(128) == 11
    assert C.outlier_capacity(64) == 5


@pytest.mark.parametrize("d", [64, 128])
def test_k_equal_channels_threshold_is_tight(d):
    # k channels with norm a, D-k with norm 0: flagged iff D - k >= 10.24 k, i.e. k <= cap
    cap = C.outlier_capacity(d)
    for k in range(1, cap + 3):
        x = np.zeros((3, d))
        x[:, :k] = 2.0
        o = C.fp4_calibrate(x)
        if k <= cap:
            assert o.tolist() == list(range(k)), k
        else:
            assert len(o) == 0, k


def test_planted_channel_closed_form():
    # 127 channels of RMS 1 and one of RMS 20: mu = 147/128, sigma^2 = 527/128 - mu^2
    x = np.ones((16, 128))
    x[:, 77] = 20.0
    x[::2] *= -1  # signs do not change RMS
    mu = 147 / 128
    sigma = np.sqrt(527 / 128 - mu ** 2)
    assert 1.0 < mu + 3.2 * sigma < 20.0
    assert C.fp4_calibrate(x).tolist() == [77]


def test_sigma_zero_gives_no_outliers():
    assert len(C.fp4_calibrate(np.full((4, 128), 0.75))) == 0
    assert len(C.fp4_calibrate(np.zeros((1, 64)))) == 0


def test_single_token_rms_is_abs():
    x = np.zeros((1, 128))
    x[0, 5] = -9.0
    x[0, 6:] = 0.1
    assert C.fp4_calibrate(x).tolist() == [5]


def test_cantelli_bound_holds_on_heavy_tails():
    rng = np.random.default_rng(0)
    for _ in range(300):
        x = rng.standard_cauchy((rng.integers(1, 17), 128)) * rng.uniform(0.1, 10)
        assert len(C.fp4_calibrate(x)) <= 11


def test_fp4_row_invariants():
    rng = np.random.default_rng(1)
    for _ in range(200):
        x = F.bf16_decode(_bf16_bits(rng.standard_normal(128) * rng.uniform(0.01, 50)))
        o = np.sort(rng.choice(128, size=rng.integers(0, 4), replace=False))
        packed, s, ov = C.fp4_encode_row(x, o)
        codes = np.empty(128, dtype=np.uint8)
        codes[0::2], codes[1::2] = packed & 0xF, packed >> 4
        inl = np.setdiff1d(np.arange(128), o)
        amax = inl[np.argmax(np.abs(x[inl]))]
        # the inlier absmax lands on +-6, outlier positions hold +0
        assert codes[amax] & 7 == 7
        assert np.all(codes[o] == 0)
        assert np.float32(s) == np.float32(np.abs(x[inl]).max()) / np.float32(6.0)
        assert np.array_equal(F.f16_decode(ov), x[o])  # bf16 values are exact in fp16 here
        # dequant error: at most half the E2M1 spacing at the scaled value (plus the
        # fp32 rounding of the quotient)
        v = x[inl] / float(s)
        deq = F.e2m1_decode(codes[inl]) * float(s)
        half = np.where(np.abs(v) < 2, 0.25, np.where(np.abs(v) < 4, 0.5, 1.0))
        assert np.all(np.abs(deq - x[inl]) <= (half + 1e-6) * float(s))


def test_fp4_zero_row():
    packed, s, ov = C.fp4_encode_row(np.zeros(128), np.zeros(0, dtype=np.int64))
    assert s == 0 and np.all(packed == 0)
    x = np.zeros(128)
    x[3] = -0.0
    packed, s, _ = C.fp4_encode_row(x, np.zeros(0, dtype=np.int64))
    assert np.all(packed == 0)  # s = 0 gives +0 codes


def test_fp8_head_scale_invariant():
    rng = np.random.default_rng(2)
    rows = _bf16_bits(rng.standard_normal((50, 4, 64)) * np.array([1, 3, 0.01, 100])[None, :, None])
    s = C.fp8_head_scale(rows, "bf16")
    x = F.bf16_decode(rows)
    for h in range(4):
        a = np.abs(x[:, h, :]).max()
        assert s[h] == np.float32(a) / np.float32(448.0)
        code = F.e4m3_encode(F.f32_quotient(np.array([a, -a]), s[h]))
        assert code.tolist() == [0x7E, 0xFE]


def _write_and_read(kind, act, rows_k, rows_v, slots, nb=8, **kw):
    hkv, d = rows_k.shape[1], rows_k.shape[2]
    pool = C.Pool.filled(kind, nb, hkv, d)
    before = {n: a.copy() for n, a in pool.arrays.items()}
    C.cache_write(pool, rows_k, rows_v, act, slots, **kw)
    return pool, before


def test_slot_placement_and_sentinels_copy_path():
    rng = np.random.default_rng(3)
    T, hkv, d = 11, 2, 64
    k = rng.integers(0, 2 ** 16, (T, hkv, d), dtype=np.uint16)
    v = rng.integers(0, 2 ** 16, (T, hkv, d), dtype=np.uint16)
    slots = rng.choice(8 * 16, T, replace=False).astype(np.int64)
    slots[4] = -1  # skipped
    pool, before = _write_and_read("f16", "f16", k, v, slots)
    written = np.zeros((8, hkv, 16), dtype=bool)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        b, o = divmod(int(s), 16)
        assert np.array_equal(pool.arrays["k"][b, :, o, :], k[i])
        assert np.array_equal(pool.arrays["v"][b, :, o, :], v[i])
        written[b, :, o] = True
    for n in ("k", "v"):
        assert np.array_equal(pool.arrays[n][~written], before[n][~written])  # sentinels


def test_distinct_slots_required():
    k = np.zeros((2, 1, 64), dtype=np.uint16)
    with pytest.raises(AssertionError):
        _write_and_read("f16", "f16", k, k, np.array([5, 5]))


def test_fp8_write_dequant_error_bound():
    rng = np.random.default_rng(4)
    T, hkv, d = 40, 2, 128
    k = _bf16_bits(rng.standard_normal((T, hkv, d)))
    v = _bf16_bits(rng.standard_normal((T, hkv, d)) * 3)
    ks, vs = C.fp8_head_scale(k, "bf16"), C.fp8_head_scale(v, "bf16")
    slots = rng.permutation(8 * 16)[:T].astype(np.int64)
    pool, before = _write_and_read("fp8", "bf16", k, v, slots, k_scale=ks, v_scale=vs)
    kd, vd = C.dequant_slot_rows(pool, slots // 16, slots % 16, ks, vs)
    for x_bits, deq, s in ((k, kd, ks), (v, vd, vs)):
        x = F.bf16_decode(x_bits)
        a = np.abs(x / s[None, :, None])
        e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
        # half the E4M3 spacing at x/s, plus the fp32 rounding of the quotient x/s
        # (the code is E4M3 of the fp32 quotient, so a quotient that rounds onto a tie
        # may land a full half-spacing plus one fp32 ulp away)
        bound = (2.0 ** (e - 4) + a * 2.0 ** -23) * s[None, :, None]
        assert np.all(np.abs(deq - x) <= bound)
    # zero scale gives +0 codes
    pool, _ = _write_and_read("fp8", "bf16", k, v, slots, k_scale=np.zeros(hkv, np.float32),
                              v_scale=vs)
    assert np.all(pool.arrays["k"][slots // 16, :, slots % 16, :] == 0)


def test_fp4_calibrates_once_per_block_and_reuses():
    rng = np.random.default_rng(5)
    d, hkv = 128, 1
    x1 = rng.standard_normal((4, hkv, d))
    x1[:, 0, 9] *= 20
    x2 = rng.standard_normal((4, hkv, d))
    x2[:, 0, 50] *= 20  # a different channel would be flagged if recalibrated
    k1, k2 = _bf16_bits(x1), _bf16_bits(x2)
    pool = C.Pool.filled("fp4", 4, hkv, d)
    C.cache_write(pool, k1, k1, "bf16", np.array([32, 33, 34, 35]))  # block 2, offsets 0-3
    rec = C.fp4_records(pool, "k")[2, 0].copy()
    assert rec[0] == 1 and rec[1] == 9 and np.all(rec[2:] == 0xFF)
    C.cache_write(pool, k2, k2, "bf16", np.array([36, 37, 38, 39]))
    assert np.array_equal(C.fp4_records(pool, "k")[2, 0], rec)  # reused, not recomputed
    kd, _ = C.dequant_slot_rows(pool, np.full(8, 2), np.arange(8))
    xall = F.bf16_decode(np.concatenate([k1, k2]))
    # the outlier channel comes back exactly (fp16 holds bf16 values exactly)
    assert np.array_equal(kd[:, 0, 9], xall[:, 0, 9])
    # untouched offsets (codes, scales, first-outlier values), the unused outlier slots
    # and the tile's padding keep their sentinel bytes
    byte, shift = C.fp4_code_map("k", d)
    assert np.array_equal(C.fp4_get_codes(pool, "k")[2, 0, 8:], (0xA5 >> shift[8:]) & 0xF)
    assert np.all(C.fp4_scales(pool, "k")[2, 0, 8:].view(np.uint8) == 0xA5)
    assert np.all(C.fp4_slot0(pool, "k")[2, 0, 8:] == 0xA5A5)
    assert np.all(pool.arrays["k_out_val"][2, 0].view(np.uint8) == 0xA5)
    assert np.all(pool.arrays["k"][2, 0, 16 * d // 2 + 112:] == 0xA5)
    assert np.all(C.fp4_records(pool, "k")[[0, 1, 3]] == 0xFF)


def test_fp4_calibration_uses_only_the_calls_tokens_in_the_block():
    d = 128
    x = np.ones((3, 1, d))
    x[0, 0, 10] = 30.0  # token in block 0
    x[1, 0, 20] = 30.0  # token in block 1
    x[2, 0, 21] = 30.0  # token in block 1
    bits = _bf16_bits(x)
    pool = C.Pool.filled("fp4", 2, 1, d)
    C.cache_write(pool, bits, bits, "bf16", np.array([3, 16, 17]))
    assert C.fp4_records(pool, "k")[0, 0, :2].tolist() == [1, 10]
    assert C.fp4_records(pool, "k")[1, 0, :3].tolist() == [2, 20, 21]


def test_fp8_code_is_e4m3_of_the_fp32_quotient():
    # The reading: the quantizer divides in fp32 (correctly rounded) and rounds that fp32
    # value to E4M3. Here x = 3.046875 (a bf16 value) and s = fp32 bits 0x3C149249: the
    # exact quotient is slightly above the tie 336 (between 320 and 352), but its fp32
    # rounding is exactly 336.0, so the code is the even neighbour 320 (0x7A), not 352.
    from fractions import Fraction
    s = np.array([0x3C149249], dtype=np.uint32).view(np.float32)[0]
    x = 3.046875
    assert Fraction(x) / Fraction(float(s)) > 336
    q = F.f32_quotient(x, s)
    assert q == 336.0
    assert int(F.e4m3_encode(q)) == 0x7A
    pool = C.Pool.filled("fp8", 1, 1, 64)
    row = np.zeros((1, 1, 64), dtype=np.uint16)
    row[0, 0, 0] = _bf16_bits(np.array([x]))[0]
    C.cache_write(pool, row, row, "bf16", np.array([0]), k_scale=np.array([s]), v_scale=np.array([s]))
    assert pool.arrays["k"][0, 0, 0, 0] == 0x7A


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kv", ["k", "v"])
def test_fp4_code_map_is_a_bijection_onto_the_code_bytes(kv, d):
    """Every (token, channel) code owns its own nibble of the 8 d code bytes, and every
    nibble belongs to one code."""
    byte, shift = C.fp4_code_map(kv, d)
    nib = (byte * 2 + shift // 4).ravel()
    assert nib.min() == 0 and nib.max() == 16 * d - 1
    assert len(np.unique(nib)) == 16 * d


@pytest.mark.parametrize("d", [64, 128])
def test_fp4_v_chunks_hold_a_channel_group_of_four_tokens(d):
    """V chunk (g, j): 2 nc bytes (nc = d / 16 channels: 16 bytes at d = 128, 8 at d = 64)
    holding channels nc g .. nc g + nc - 1 of tokens 4 j .. 4 j + 3, two tokens per byte
    (one channel), so a converter taking a byte yields a token pair."""
    nc = d // 16
    byte, shift = C.fp4_code_map("v", d)
    for g in range(d // nc):
        for j in range(4):
            chunk = g * 4 + j
            t = np.arange(4 * j, 4 * j + 4)[:, None]
            ch = np.arange(nc * g, nc * g + nc)[None, :]
            b = byte[t, ch]
            assert np.all(b // (2 * nc) == chunk)
            # one byte = one channel, two consecutive tokens (even token low)
            for c in range(nc):
                col = b[:, c]
                assert col[0] == col[1] and col[2] == col[3] and col[0] + 1 == col[2]
                assert col[0] % (2 * nc) == 2 * c
                assert list(shift[t[:, 0], ch[0, c]]) == [0, 4, 0, 4]


@pytest.mark.parametrize("d", [64, 128])
def test_fp4_put_codes_keeps_the_other_nibbles(d):
    for kv in ("k", "v"):
        pool = C.Pool.filled("fp4", 2, 1, d)
        rng = np.random.default_rng(3)
        want = np.full((16, d), -1)
        for t in rng.permutation(16)[:7]:
            codes = rng.integers(0, 16, d).astype(np.uint8)
            C.fp4_put_codes(pool, kv, 1, 0, int(t), codes)
            want[t] = codes
        got = C.fp4_get_codes(pool, kv)[1, 0]
        byte, shift = C.fp4_code_map(kv, d)
        sentinel = (0xA5 >> shift) & 0xF
        assert np.array_equal(got, np.where(want >= 0, want, sentinel))
        assert np.all(C.fp4_code_bytes(pool, kv)[0] == 0xA5)


@pytest.mark.parametrize("kind", ["fp8t", "bf8t"])
def test_fp8_token_scale_pool_invariants(kind):
    """Per-token FP8: every written row's largest magnitude encodes to the format's largest
    code, dequantized values are within half a grid step (times the scale) of the input,
    and every byte of unwritten rows keeps its sentinel."""
    fmt = C.FP8_KINDS[kind][0]
    top = 0x7E if fmt == "e4m3" else 0x7B
    rng = np.random.default_rng(4)
    d, hkv, nb = 128, 2, 4
    x = rng.standard_normal((10, hkv, d)).astype(np.float32) * 3
    x[:, 0, 7] *= 20
    bits = ((x.view(np.uint32) + 0x7FFF + ((x.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)
    pool = C.Pool.filled(kind, nb, hkv, d)
    slots = np.array([16 + 3, 16 + 9, 48, 49, 50, 51, 52, 53, 54, 55], dtype=np.int64)
    C.cache_write(pool, bits, bits, "bf16", slots)
    xv = F.bf16_decode(bits)
    codes = C.fp8t_codes(pool, "k")
    sc = C.fp8t_scales(pool, "k")
    blk, off = slots // 16, slots % 16
    for i in range(len(slots)):
        for h in range(hkv):
            c = codes[blk[i], h, off[i]]
            j = int(np.argmax(np.abs(xv[i, h])))
            assert (int(c[j]) & 0x7F) == top
            assert sc[blk[i], h, off[i]] == np.float32(np.abs(xv[i, h]).max() / F.fp8_max(fmt))
    kd, vd = C.dequant_slot_rows(pool, blk, off)
    mags = F.e4m3_magnitudes() if fmt == "e4m3" else F.e5m2_magnitudes()
    step = np.max(np.diff(mags) / np.maximum(mags[1:], 1e-300))  # relative grid step bound
    s = sc[blk, :, off][..., None].astype(np.float64)
    assert np.all(np.abs(kd - xv) <= np.maximum(np.abs(xv) * step, s * mags[1]) + 1e-12)
    # V rows are the K rows here, so V's token scales equal K's; both sets sit in the K run
    # (K's at 16 D, V's at 16 D + 64) and the V run holds codes only
    sv = C.fp8t_scales(pool, "v")
    assert np.array_equal(sv[blk, :, off], sc[blk, :, off])
    assert pool.arrays["k"].shape[-1] == 16 * d + 128 and pool.arrays["v"].shape[-1] == 16 * d
    # untouched rows: offsets other than the written ones, and blocks 0 and 2 entirely
    raw = pool.arrays["k"]
    assert np.all(raw[[0, 2]] == 0xA5)
    assert np.all(pool.arrays["v"][[0, 2]] == 0xA5)
    assert np.all(codes[1, :, [o for o in range(16) if o not in (3, 9)]] == 0xA5)
    assert np.all(raw[3, :, 16 * d + 32:16 * d + 64] == 0xA5)  # K scales of offsets 8..15
    assert np.all(raw[3, :, 16 * d + 96:] == 0xA5)  # V scales of offsets 8..15


def test_fp8_head_scale_e5m2_invariant():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((50, 3, 64)) * 7).astype(np.float16).view(np.uint16)
    s = C.fp8_head_scale(x, "f16", "e5m2")
    pool = C.Pool.filled("bf8", 4, 3, 64)
    C.cache_write(pool, x[:16], x[:16], "f16", np.arange(16, 32), s, s)
    xv = F.f16_decode(x[:16])
    for h in range(3):
        if np.abs(xv[:, h]).max() == np.abs(F.f16_decode(x)[:, h]).max():
            j = np.unravel_index(np.argmax(np.abs(xv[:, h])), xv[:, h].shape)
            assert int(pool.arrays["k"][1, h, j[0], j[1]]) & 0x7F == 0x7B


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_v_run_layout_by_channel(d):
    """FP8 V runs hold their codes by channel, in 16-byte slots (piece, token four, channel
    group): the byte order, written out as nested loops, equals fp8_v_byte; it is a
    permutation of the run; and writing rows then reading them back gives the rows."""
    nt = d // 16
    want = np.empty((16, d), dtype=np.int64)
    pos = 0
    for piece in range(nt // 4):
        for q in range(4):
            for g in range(16):
                for jj in range(4):
                    for r in range(4):
                        want[4 * q + r, nt * g + 4 * piece + jj] = pos
                        pos += 1
    got = C.fp8_v_byte(np.arange(16)[:, None], np.arange(d)[None, :], d)
    assert np.array_equal(got, want)
    assert np.array_equal(np.sort(got.ravel()), np.arange(16 * d))
    rng = np.random.default_rng(7)
    for kind in ("fp8", "fp8t"):
        pool = C.Pool.filled(kind, 3, 2, d)
        blk = np.array([2, 0, 2, 1])
        off = np.array([5, 15, 0, 7])
        rows = rng.integers(0, 256, (4, 2, d), dtype=np.uint8)
        C.fp8_put_codes(pool, "v", blk, off, rows)
        assert np.array_equal(C.fp8_get_codes(pool, "v", blk, off), rows)
        run = pool.arrays["v"].reshape(3, 2, -1)
        assert run[2, 1, C.fp8_v_byte(5, d - 1, d)] == rows[0, 1, d - 1]
        # the K run keeps token rows
        C.fp8_put_codes(pool, "k", blk, off, rows)
        krun = pool.arrays["k"].reshape(3, 2, -1)
        assert np.array_equal(krun[0, 1, 15 * d:16 * d], rows[1, 1])


@pytest.mark.parametrize("d", [64, 128])
def test_header_fp8_v_byte_macro_matches_oracle(d, tmp_path):
    """The public header's PA_FP8_V_BYTE, compiled with the host C compiler, gives the
    oracle's byte offset for every (token, channel) of a run."""
    import os
    import shutil
    import subprocess
    from conftest import ROOT
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    src = tmp_path / "v.c"
    src.write_text('#include <stdio.h>\n#include "pa.h"\nint main(void) {\n'
                   f'  for (int t = 0; t < 16; ++t) for (int c = 0; c < {d}; ++c)\n'
                   f'    printf("%d\\n", PA_FP8_V_BYTE(t, c, {d}));\n  return 0;\n}}\n')
    exe = tmp_path / "v"
    subprocess.run([cc, "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o",
                    str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    got = np.array(out.split(), dtype=np.int64).reshape(16, d)
    want = C.fp8_v_byte(np.arange(16)[:, None], np.arange(d)[None, :], d)
    assert np.array_equal(got, want)
