"""Pins of the oracle's per-sequence FP4 calibration (fp4_sequence_records and the
seq_records path of cache_write).

The outlier set of a sequence comes from the per-channel RMS norms of its first prefill
chunk, with the same mean + 3.2 sigma rule as the per-block calibration. Pinned by: a
pure-Python recomputation of the statistics on small rows; planted channels known a priori;
blocks opened later (a decode token that starts a fresh block) taking the sequence's set
rather than one computed from their own few tokens; each of two sequences with different
planted channels keeping its own set; and the stored values at outlier channels being the
inputs rounded to fp16."""
import math

import numpy as np

from oracle import cache as C
from oracle.formats import act_decode, f16_decode

D, HKV = 128, 2


def _bf16_bits(x):
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _brute_set(x):
    """mean + 3.2 sigma over per-channel RMS, with Python floats and loops."""
    n, d = len(x), len(x[0])
    r = [math.sqrt(sum(x[t][c] * x[t][c] for t in range(n)) / n) for c in range(d)]
    mu = sum(r) / d
    sd = math.sqrt(sum((v - mu) ** 2 for v in r) / d)
    if sd == 0.0:
        return []
    return [c for c in range(d) if r[c] >= mu + 3.2 * sd]


def test_sequence_records_match_brute_force_statistics():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((40, HKV, D)).astype(np.float32)
    x[:, 0, 17] *= 9.0
    x[:, 1, [3, 100]] *= 6.0
    kb = _bf16_bits(x)
    vb = _bf16_bits(x[::-1] * 0.5)
    recs, margins = C.fp4_sequence_records(kb, vb, "bf16", [0, 25, 40])
    for side, bits in enumerate((kb, vb)):
        for sq, (a, b) in enumerate(((0, 25), (25, 40))):
            xv = act_decode(bits[a:b], "bf16")
            for h in range(HKV):
                want = _brute_set(xv[:, h, :].tolist())
                rec = recs[sq, side, h]
                assert rec[0] == len(want)
                assert rec[1:1 + rec[0]].tolist() == want
                assert (rec[1 + rec[0]:] == 0xFF).all()
                assert margins[sq, side, h] > 1e-3
    assert recs[0, 0, 0, :2].tolist() == [1, 17]
    assert recs[0, 0, 1, :3].tolist() == [2, 3, 100]


def test_empty_sequence_has_no_outliers():
    kb = _bf16_bits(np.ones((4, HKV, D), dtype=np.float32))
    recs, _ = C.fp4_sequence_records(kb, kb, "bf16", [0, 0, 4])
    assert (recs[0, :, :, 0] == 0).all()
    assert (recs[1, :, :, 0] == 0).all()  # constant rows: sigma = 0 -> no outliers


def _two_sequences():
    """Two sequences of 65 and 49 tokens: each one's last token opens a fresh block."""
    rng = np.random.default_rng(2)
    lens = [65, 49]
    b1 = lens[0]
    x = rng.standard_normal((2, sum(lens), HKV, D)).astype(np.float32)
    x[:, :b1, :, 11] *= 20.0        # sequence 0: channel 11
    x[:, b1:, :, 90] *= 20.0        # sequence 1: channel 90
    x[:, b1 + 48, :, 90] = 0.1      # ... whose last token peaks elsewhere
    x[:, b1 + 48, :, 40] = 15.0
    kb, vb = _bf16_bits(x[0]), _bf16_bits(x[1])
    token_seq = np.repeat([0, 1], lens)
    # first prefill chunk: 32 tokens of each sequence
    k_first = np.concatenate([kb[0:32], kb[b1:b1 + 32]])
    v_first = np.concatenate([vb[0:32], vb[b1:b1 + 32]])
    recs, _ = C.fp4_sequence_records(k_first, v_first, "bf16", [0, 32, 64])
    tables = np.array([[5, 0, 7, 2, 9], [3, 8, 1, 4, -1]], dtype=np.int32)
    return lens, kb, vb, token_seq, recs, tables


def _slots(tables, s, pos):
    pos = np.asarray(pos)
    return tables[s, pos // 16].astype(np.int64) * 16 + pos % 16


def test_blocks_take_their_sequence_set_including_fresh_decode_blocks():
    lens, kb, vb, token_seq, recs, tables = _two_sequences()
    assert recs[0, 0, 0, :2].tolist() == [1, 11] and recs[1, 1, 1, :2].tolist() == [1, 90]
    pool = C.Pool.filled("fp4", 10, HKV, D)
    blk_pool = C.Pool.filled("fp4", 10, HKV, D)
    # prefill in chunks of 16 tokens, all but the last token of each sequence
    for s, L in enumerate(lens):
        base = sum(lens[:s])
        for lo in range(0, L - 1, 16):
            pos = np.arange(lo, min(lo + 16, L - 1))
            rows = base + pos
            sl = _slots(tables, s, pos)
            C.cache_write(pool, kb[rows], vb[rows], "bf16", sl, seq_records=recs,
                          token_seq=token_seq[rows])
            C.cache_write(blk_pool, kb[rows], vb[rows], "bf16", sl)
    # decode step: position 64 opens block 4 of sequence 0 and position 48 block 3 of
    # sequence 1, one token each
    rows = np.array([64, lens[0] + 48])
    sl = np.concatenate([_slots(tables, 0, [64]), _slots(tables, 1, [48])])
    C.cache_write(pool, kb[rows], vb[rows], "bf16", sl, seq_records=recs, token_seq=token_seq[rows])
    C.cache_write(blk_pool, kb[rows], vb[rows], "bf16", sl)
    for s, L in enumerate(lens):
        for j in range(-(-L // 16)):
            b = tables[s, j]
            for side, name in enumerate("kv"):
                got = C.fp4_records(pool, name)[b]
                assert np.array_equal(got, recs[s, side]), (s, j, name)
    # under the per-block reading that one-token block flags its own token's peak instead
    one = C.fp4_records(blk_pool, "k")[tables[1, 3], 0]
    assert one[:2].tolist() == [1, 40]


def test_seq_mode_values_at_outlier_channels_are_fp16_of_the_inputs():
    lens, kb, vb, token_seq, recs, tables = _two_sequences()
    pool = C.Pool.filled("fp4", 10, HKV, D)
    rows = np.arange(lens[0], lens[0] + lens[1])
    sl = _slots(tables, 1, np.arange(lens[1]))
    C.cache_write(pool, kb[rows], vb[rows], "bf16", sl, seq_records=recs, token_seq=token_seq[rows])
    kd, vd = C.dequant_slot_rows(pool, sl // 16, sl % 16)
    x = act_decode(kb[rows], "bf16")
    for h in range(HKV):
        cnt = recs[1, 0, h, 0]
        for c in recs[1, 0, h, 1:1 + cnt]:
            want = f16_decode(np.asarray(x[:, h, c], dtype=np.float16).view(np.uint16))
            assert np.array_equal(kd[:, h, c], want)
    # inliers: E2M1 steps are at most 2 at scale 1 (between 4 and 6), so rounding moves a
    # value by at most 1 step-half = s_t = max inlier |x| / 6
    for h in range(HKV):
        o = set(recs[1, 0, h, 1:1 + recs[1, 0, h, 0]].tolist())
        inl = [c for c in range(D) if c not in o]
        amax = np.abs(x[:, h, inl]).max(axis=1)
        assert (np.abs(kd[:, h, inl] - x[:, h, inl]).max(axis=1) <= amax / 6 + 1e-12).all()
