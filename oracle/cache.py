"""Paged KV pool: cache-write replay, dequantization and block-table gather (fp64, CPU).

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg may import this package.

What the pages fix:
  * KV lives in fixed physical blocks of 16 tokens, reached through a per-sequence
    logical->physical block table (inferensys glossary "vLLM", PagedAttention entry;
    xonoai.com field report on vLLM v0.7.2, "Deconstructing the v0.7.2 Architecture",
    and its launch flag --block-size 16).
  * FP8 E4M3 KV quantization with a fp32 scale (xonoai.com report, same section).
  * 4-bit outlier-aware quantization (dailyaiworld.com, "vLLM 0.7 Ships Unified KV
    Cache Compression", "Technical Breakdown: Dynamic Quantization with Outlier
    Retention", steps 1-3): per-channel magnitude norms, channels at or above a 3.2 sigma
    threshold kept in an fp16 outlier buffer, the remaining channels normalized and
    quantized to FP4.

Readings where the pages are silent (each listed in the design notes):
  * FP8: code = E4M3(fp32(x / s_h)); the quotient is the correctly rounded fp32 one and
    that fp32 value is rounded to E4M3 (nearest, ties even, saturating). s_h is the
    per-(layer, kv-head) fp32 scale fp32(absmax_h / 448), absmax over every value of that
    head the run writes, K and V separately. s = 0 gives +0 codes.
  * FP4 calibration granularity: per (physical block, kv-head, K|V), on the tokens the
    first write into that block carries; later writes reuse the stored channel set.
    The per-channel norm is the RMS over those tokens; mu and sigma are the mean and
    population standard deviation of the D norms; outliers are the channels with
    norm >= mu + 3.2 sigma, ascending; sigma = 0 means no outliers.
    The variant closest to the pages' wording ("per-channel norms ... during the prefill
    phase") computes one set per (sequence, kv-head, K|V) from the sequence's first
    prefill chunk and gives it to every block the sequence opens (fp4_sequence_records,
    cache_write's seq_records).
  * FP4 scale: one fp32 scale per (token, kv-head, K|V), fp32(inlier absmax / 6); inlier
    codes are E2M1(fp32(x / s_t)); outlier positions hold code +0; s_t = 0 gives +0 codes;
    two codes per byte, even channel in the low nibble; outliers are stored as fp16(x).

Pool layout (the boundary's layout, one array per field):
  f16 / bf16 : k, v          uint16 [NB, Hkv, 16, D]        token rows
  fp8, bf8   : k             uint8  [NB, Hkv, 16, D]        K codes, token rows
               v             uint8  [NB, Hkv, 16, D]        V codes of a (block, head) by
                                    channel in 16-byte slots, fp8_v_byte
                                    (+ per-head fp32 scales)
  fp8t, bf8t : k             uint8  [NB, Hkv, 16 D + 128] one run per (block, head):
                 [0, 16 D)         K codes [16 tokens][D]
                 [16 D, 16 D + 64)  K per-token scales, fp32 [16]
                 [16 D + 64, 16 D + 128)  V per-token scales, fp32 [16]
               v             uint8  [NB, Hkv, 16 D]       V codes by channel, fp8_v_byte
  fp4        : k, v          uint8  [NB, Hkv, TILE] one run of bytes per (block, head):
                 [0, 8 D)          codes [16 tokens][D/2], two per byte
                 [8 D, 8 D + 64)   per-token scales, fp32 [16]
                 next 16 bytes     record: byte 0 = outlier count (0xFF = not yet
                                   calibrated), then the ascending channel indices,
                                   then 0xFF in the unused bytes
                 next 32 bytes     fp16 values of the first outlier, one per token
                 the rest          padding up to a multiple of 128 bytes (TILE = 1152
                                   for D = 128, 640 for D = 64)
               *_out_val     uint16 [NB, Hkv, CAP - 1, 16]  fp16 bits of outliers 1.. CAP-1
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .formats import (
    E4M3_MAX,
    E2M1_MAX,
    act_decode,
    e2m1_decode,
    e2m1_encode,
    e4m3_decode,
    e4m3_encode,
    f16_decode,
    fp8_decode,
    fp8_encode,
    fp8_max,
    f16_encode,
    f32_quotient,
    f32_round,
)

BLOCK_TOKENS = 16
OUTLIER_SIGMAS = 3.2
UNCALIBRATED = 0xFF


def outlier_capacity(head_dim: int) -> int:
    """Most channels that can reach mu + 3.2 sigma among head_dim norms.

    If k channels satisfy r_c - mu >= 3.2 sigma, the other head_dim - k deviations sum to
    at most -3.2 k sigma, so (Cauchy-Schwarz) D sigma^2 >= 10.24 k sigma^2 (1 + k/(D-k)),
    i.e. k <= D / (1 + 3.2^2). 11 for D = 128, 5 for D = 64."""
    return int(np.floor(head_dim / (1.0 + OUTLIER_SIGMAS ** 2)))


# FP8 pool kinds: code format and where the scale lives ("head": a per-(layer, kv head)
# input; "token": computed per (token, kv head, K|V) at write time, stored in the run)
FP8_KINDS = {"fp8": ("e4m3", "head"), "bf8": ("e5m2", "head"),
             "fp8t": ("e4m3", "token"), "bf8t": ("e5m2", "token")}


@dataclass
class Pool:
    kind: str  # "f16" | "bf16" | "fp8" | "bf8" | "fp8t" | "bf8t" | "fp4"
    num_blocks: int
    num_kv_heads: int
    head_dim: int
    arrays: dict = field(default_factory=dict)

    @staticmethod
    def shapes(kind, nb, hkv, d):
        if kind in ("f16", "bf16"):
            return {"k": ((nb, hkv, 16, d), np.uint16), "v": ((nb, hkv, 16, d), np.uint16)}
        if kind in ("fp8", "bf8"):
            return {"k": ((nb, hkv, 16, d), np.uint8), "v": ((nb, hkv, 16, d), np.uint8)}
        if kind in ("fp8t", "bf8t"):
            return {"k": ((nb, hkv, fp8t_run_bytes(d, "k")), np.uint8),
                    "v": ((nb, hkv, fp8t_run_bytes(d, "v")), np.uint8)}
        if kind == "fp4":
            cap = outlier_capacity(d)
            out = {}
            for kv in ("k", "v"):
                out[kv] = ((nb, hkv, fp4_tile_bytes(d)), np.uint8)
                out[kv + "_out_val"] = ((nb, hkv, cap - 1, 16), np.uint16)
            return out
        raise ValueError(kind)

    @classmethod
    def filled(cls, kind, nb, hkv, d, sentinel=0xA5):
        """A pool whose every byte is `sentinel`, except that FP4 calibration records
        start as 'not calibrated' (all 0xFF), which the caller must arrange."""
        p = cls(kind, nb, hkv, d)
        for name, (shape, dt) in cls.shapes(kind, nb, hkv, d).items():
            n = int(np.prod(shape)) * np.dtype(dt).itemsize
            p.arrays[name] = np.full(n, sentinel, dtype=np.uint8).view(dt).reshape(shape)
        if kind == "fp4":
            for kv in ("k", "v"):
                fp4_records(p, kv)[...] = UNCALIBRATED
        return p


# ----------------------------------------------------------------------------------
# FP4 tile regions (views into a pool's k / v byte arrays)
# ----------------------------------------------------------------------------------


def fp8t_run_bytes(head_dim: int, kv: str = "k") -> int:
    """Bytes of one per-token-scaled FP8 (block, head) run: the 16 x D code bytes (token
    rows); the K run then holds the 16 fp32 token scales of K and the 16 of V (so every
    run is a whole number of 128-byte lines)."""
    return 16 * head_dim + (128 if kv == "k" else 0)


def fp8t_codes(pool: Pool, kv: str) -> np.ndarray:
    """K codes of a per-token-scaled FP8 pool, a view [NB, Hkv, 16, D] uint8 (token rows;
    V runs store their codes by channel, see fp8_v_byte)."""
    assert kv == "k", "V codes are stored by channel: fp8_get_codes"
    d = pool.head_dim
    a = pool.arrays[kv]
    return a[..., :16 * d].reshape(a.shape[0], a.shape[1], 16, d)


def fp8_v_byte(t, ch, d):
    """Byte offset of token t (0..15), channel ch in the V code run of one (block, kv head)
    of an FP8 pool (E4M3 or E5M2, head or token scales). With nt = d / 16, channel ch is
    channel j = ch % nt of group g = ch // nt, and token t is token r = t % 4 of four
    q = t // 4. The run is d / 64 pieces of 1024 bytes; piece j // 4 holds 64 slots of 16
    bytes, slot 16 q + g holding channels 4 (j // 4) .. 4 (j // 4) + 3 of group g for the
    four tokens of four q, channel after channel, a channel's four token bytes side by
    side."""
    nt = d // 16
    g, j = ch // nt, ch % nt
    return (j // 4) * 1024 + (16 * (t // 4) + g) * 16 + (j % 4) * 4 + t % 4


def _fp8_v_offsets(d):
    t = np.arange(16)[:, None]
    ch = np.arange(d)[None, :]
    return fp8_v_byte(t, ch, d)  # [16, d]


def _fp8_runs(pool: Pool, kv: str) -> np.ndarray:
    """[NB, Hkv, 16 D] view of the code bytes of an FP8 pool's K or V runs."""
    a = pool.arrays[kv]
    d = pool.head_dim
    return a.reshape(a.shape[0], a.shape[1], -1)[..., :16 * d]


def fp8_put_codes(pool: Pool, kv: str, blk, off, codes) -> None:
    """Store code rows codes [n, Hkv, D] of tokens (blk[i], off[i]): K runs by token row,
    V runs by channel (fp8_v_byte)."""
    blk = np.asarray(blk, dtype=np.int64)
    off = np.asarray(off, dtype=np.int64)
    d = pool.head_dim
    runs = _fp8_runs(pool, kv)
    if kv == "k":
        pos = off[:, None] * d + np.arange(d)[None, :]  # [n, d]
    else:
        pos = _fp8_v_offsets(d)[off]  # [n, d]
    h = np.arange(pool.num_kv_heads)
    runs[blk[:, None, None], h[None, :, None], pos[:, None, :]] = codes


def fp8_get_codes(pool: Pool, kv: str, blk, off) -> np.ndarray:
    """Code rows [n, Hkv, D] of tokens (blk[i], off[i]), the inverse of fp8_put_codes."""
    blk = np.asarray(blk, dtype=np.int64)
    off = np.asarray(off, dtype=np.int64)
    d = pool.head_dim
    runs = _fp8_runs(pool, kv)
    if kv == "k":
        pos = off[:, None] * d + np.arange(d)[None, :]
    else:
        pos = _fp8_v_offsets(d)[off]
    h = np.arange(pool.num_kv_heads)
    return runs[blk[:, None, None], h[None, :, None], pos[:, None, :]]


def fp8t_scales(pool: Pool, kv: str) -> np.ndarray:
    """Per-token scales of K or V in a per-token-scaled FP8 pool, a view [NB, Hkv, 16]
    fp32 (both live in the K array's runs, K's first)."""
    d = pool.head_dim
    at = 16 * d + (0 if kv == "k" else 64)
    return pool.arrays["k"][..., at:at + 64].view(np.float32)


def fp4_tile_bytes(head_dim: int) -> int:
    """Bytes of one FP4 (block, head) run: codes, 16 fp32 scales, a 16-byte record and the
    first outlier's 16 fp16 values, rounded up to a multiple of 128 bytes."""
    used = 16 * head_dim // 2 + 16 * 4 + 16 + 16 * 2
    return -(-used // 128) * 128


def _fp4_offsets(d):
    codes = 16 * d // 2
    return codes, codes + 64, codes + 80, codes + 112  # scales, record, slot 0, end


def fp4_code_map(kv: str, d: int):
    """Where the 4-bit code of (token t, channel ch) sits in a run's first 8 d bytes:
    (byte index [16, d], bit shift [16, d]).

    K codes are token rows: byte t * d/2 + ch // 2, the even channel in the low nibble.
    V codes are grouped for a transposed read, in chunks of nc = d / 16 channels of four
    tokens (2 nc bytes: 16 for d = 128, 8 for d = 64): chunk (ch // nc) * 4 + t // 4 holds
    channels nc g .. nc g + nc - 1 of tokens 4 j .. 4 j + 3; inside it, channel ch % nc
    takes bytes 2 (ch % nc) and 2 (ch % nc) + 1 (tokens 0-1 and 2-3 of the four), the
    even token in the low nibble."""
    t = np.arange(16)[:, None]
    ch = np.arange(d)[None, :]
    nc = d // 16
    if kv == "k":
        byte = t * (d // 2) + ch // 2
        shift = 4 * (ch % 2)
    elif kv == "v":
        byte = ((ch // nc) * 4 + t // 4) * (2 * nc) + (ch % nc) * 2 + (t % 4) // 2
        shift = 4 * (t % 2)
    else:
        raise ValueError(kv)
    return np.broadcast_to(byte, (16, d)).copy(), np.broadcast_to(shift, (16, d)).copy()


def fp4_code_bytes(pool: Pool, kv: str) -> np.ndarray:
    """The code bytes of every run, a view [NB, Hkv, 8 D] uint8 (layout: fp4_code_map)."""
    return pool.arrays[kv][..., :8 * pool.head_dim]


def fp4_get_codes(pool: Pool, kv: str) -> np.ndarray:
    """All 4-bit codes as [NB, Hkv, 16, D] uint8 (a copy)."""
    byte, shift = fp4_code_map(kv, pool.head_dim)
    raw = fp4_code_bytes(pool, kv)
    return ((raw[..., byte] >> shift.astype(np.uint8)) & 0xF).astype(np.uint8)


def fp4_put_codes(pool: Pool, kv: str, blk: int, h: int, t: int, codes: np.ndarray) -> None:
    """Store the D codes of token t of run (blk, h); the other tokens' nibbles stay."""
    byte, shift = fp4_code_map(kv, pool.head_dim)
    raw = fp4_code_bytes(pool, kv)[blk, h]
    b, sh = byte[t], shift[t].astype(np.uint8)
    clear = np.zeros(raw.shape, dtype=np.uint8)
    put = np.zeros(raw.shape, dtype=np.uint8)
    np.bitwise_or.at(clear, b, np.uint8(0xF) << sh)  # a byte may hold two of the nibbles
    np.bitwise_or.at(put, b, np.asarray(codes, dtype=np.uint8) << sh)
    raw[:] = (raw & ~clear) | put


def fp4_scales(pool: Pool, kv: str) -> np.ndarray:
    """Per-token scales, a view [NB, Hkv, 16] fp32."""
    s0, r0, _, _ = _fp4_offsets(pool.head_dim)
    return pool.arrays[kv][..., s0:r0].view(np.float32)


def fp4_records(pool: Pool, kv: str) -> np.ndarray:
    """Outlier records, a view [NB, Hkv, 16] uint8."""
    _, r0, z0, _ = _fp4_offsets(pool.head_dim)
    return pool.arrays[kv][..., r0:z0]


def fp4_slot0(pool: Pool, kv: str) -> np.ndarray:
    """fp16 bits of the first outlier, a view [NB, Hkv, 16] uint16."""
    _, _, z0, e0 = _fp4_offsets(pool.head_dim)
    return pool.arrays[kv][..., z0:e0].view(np.uint16)


def fp4_outlier_values(pool: Pool, kv: str, blk, h) -> np.ndarray:
    """All CAP outlier slots of one (block, head) as fp16 bits [CAP, 16] (a copy)."""
    return np.concatenate([fp4_slot0(pool, kv)[blk, h][None, :],
                           pool.arrays[kv + "_out_val"][blk, h]], axis=0)


# ----------------------------------------------------------------------------------
# scales
# ----------------------------------------------------------------------------------


def fp8_head_scale(rows_bits: np.ndarray, act: str, fmt: str = "e4m3") -> np.ndarray:
    """Per-kv-head fp32 scale fp32(absmax_h / max) over rows [T, Hkv, D], max = 448 (E4M3)
    or 57344 (E5M2) (the rows are visited in slices only to bound memory; a maximum does
    not depend on order)."""
    absmax = np.zeros(rows_bits.shape[1])
    for lo in range(0, rows_bits.shape[0], 1 << 16):
        x = act_decode(rows_bits[lo:lo + (1 << 16)], act)
        absmax = np.maximum(absmax, np.abs(x).max(axis=(0, 2)))
    return f32_quotient(absmax, fp8_max(fmt)).astype(np.float32)


def fp8_token_scale(x: np.ndarray, fmt: str) -> np.ndarray:
    """Per-row fp32 scale fp32(max_c |x_c| / max) of rows x [..., D] (fp64 of the input
    values): the scale each token's row is quantized with when it is written (dynamic,
    per token, the FP8 counterpart of the 4-bit path's per-token scale)."""
    return f32_quotient(np.abs(x).max(axis=-1), fp8_max(fmt))


# ----------------------------------------------------------------------------------
# FP4 pieces
# ----------------------------------------------------------------------------------


def fp4_calibrate(x: np.ndarray) -> np.ndarray:
    """Outlier channel set of one (block, head) from its tokens x [n, D] (fp64).

    Per-channel RMS norm over the n tokens, then every channel whose norm is at least
    mean + 3.2 * population-std of the D norms; ascending. sigma = 0 -> none."""
    r = np.sqrt(np.mean(x * x, axis=0))
    mu = np.mean(r)
    sigma = np.sqrt(np.mean((r - mu) ** 2))
    if sigma == 0.0:
        return np.zeros(0, dtype=np.int64)
    return np.nonzero(r >= mu + OUTLIER_SIGMAS * sigma)[0].astype(np.int64)


def fp4_calibration_margin(x: np.ndarray) -> float:
    """Smallest |r_c - threshold| / threshold of the calibration above (inf if sigma=0);
    used to flag near-ties where fp32 and fp64 statistics may disagree."""
    r = np.sqrt(np.mean(x * x, axis=0))
    mu = np.mean(r)
    sigma = np.sqrt(np.mean((r - mu) ** 2))
    if sigma == 0.0:
        return np.inf
    thr = mu + OUTLIER_SIGMAS * sigma
    return float(np.min(np.abs(r - thr)) / thr)


def fp4_sequence_records(k_rows, v_rows, act: str, row_start) -> tuple:
    """Per-sequence outlier sets (the calibration read literally: the per-channel norms of
    the key and value vectors a sequence's prefill produces, here its first prefill chunk).

    k_rows, v_rows [R, Hkv, D] raw 16-bit bits; sequence s owns rows row_start[s] ..
    row_start[s + 1] - 1. Returns (records [S, 2, Hkv, 16] uint8 in the block record format
    - count, ascending channel ids, 0xFF padding; side 0 = K, 1 = V - and margins [S, 2, Hkv]
    as in fp4_calibration_margin). A sequence with no rows gets an empty set."""
    row_start = np.asarray(row_start, dtype=np.int64)
    S = len(row_start) - 1
    hkv = np.asarray(k_rows).shape[1]
    recs = np.full((S, 2, hkv, 16), UNCALIBRATED, dtype=np.uint8)
    margins = np.full((S, 2, hkv), np.inf)
    for side, rows in enumerate((k_rows, v_rows)):
        for sq in range(S):
            x = act_decode(np.asarray(rows)[row_start[sq]:row_start[sq + 1]], act)  # [n, Hkv, D]
            for h in range(hkv):
                if x.shape[0] == 0:
                    recs[sq, side, h, 0] = 0
                    continue
                o = fp4_calibrate(x[:, h, :])
                margins[sq, side, h] = fp4_calibration_margin(x[:, h, :])
                recs[sq, side, h, 0] = len(o)
                recs[sq, side, h, 1:1 + len(o)] = o
    return recs, margins


def fp4_encode_row(x: np.ndarray, outliers: np.ndarray):
    """One token row x [D] (fp64 of the input values) with its block's outlier set.

    Returns (packed codes [D/2] uint8, fp32 scale, fp16 outlier bits [len(outliers)])."""
    d = x.shape[0]
    inlier = np.ones(d, dtype=bool)
    inlier[outliers] = False
    a = np.abs(x[inlier]).max() if inlier.any() else 0.0
    s = float(f32_quotient(a, E2M1_MAX))
    codes = np.zeros(d, dtype=np.uint8)
    if s != 0.0:
        codes[inlier] = e2m1_encode(f32_quotient(x[inlier], s))
    packed = (codes[0::2] | (codes[1::2] << np.uint8(4))).astype(np.uint8)
    return packed, np.float32(s), f16_encode(x[outliers])


# ----------------------------------------------------------------------------------
# the write
# ----------------------------------------------------------------------------------


def cache_write(pool: Pool, k_rows, v_rows, act: str, slots, k_scale=None, v_scale=None,
                only_blocks=None, calib_log=None, seq_records=None, token_seq=None):
    """Replay one cache-write call: row i of k_rows/v_rows [T, Hkv, D] (raw 16-bit bits)
    goes to slot slots[i] = physical_block * 16 + offset; negative slots are skipped.

    Slots within one call must be distinct. If only_blocks is given, only writes into
    those physical blocks are replayed (each block's contents depend only on the calls
    that write into it, so sampled replays are exact). If calib_log is a list, every FP4
    calibration appends (name, block, head, margin) with margin as in
    fp4_calibration_margin.

    FP4 per-sequence calibration: with seq_records [S, 2, Hkv, 16] (fp4_sequence_records)
    and token_seq [T] (the sequence of each row), a block this call opens takes the record
    of the sequence of its lowest-offset row in the call instead of calibrating on the
    call's rows; blocks already calibrated keep their record either way."""
    slots = np.asarray(slots, dtype=np.int64)
    live = np.nonzero(slots >= 0)[0]
    assert len(np.unique(slots[live])) == len(live), "slots within one call must be distinct"
    if only_blocks is not None:
        keep = np.isin(slots[live] // BLOCK_TOKENS, np.asarray(list(only_blocks)))
        live = live[keep]
    blk = slots[live] // BLOCK_TOKENS
    off = slots[live] % BLOCK_TOKENS
    assert (blk < pool.num_blocks).all()
    A = pool.arrays
    if pool.kind in ("f16", "bf16"):
        assert pool.kind == act, "a 16-bit pool stores the activation dtype unchanged"
        A["k"][blk, :, off, :] = np.asarray(k_rows)[live]
        A["v"][blk, :, off, :] = np.asarray(v_rows)[live]
        return
    if pool.kind in FP8_KINDS:
        fmt, where = FP8_KINDS[pool.kind]
        for name, rows, sc in (("k", k_rows, k_scale), ("v", v_rows, v_scale)):
            x = act_decode(np.asarray(rows)[live], act)  # [n, Hkv, D]
            if where == "head":
                s = np.asarray(sc, dtype=np.float32).astype(np.float64)[None, :, None]
            else:
                s = fp8_token_scale(x, fmt)[..., None]  # [n, Hkv, 1]
            q = f32_quotient(x, s)
            codes = fp8_encode(np.where(s == 0.0, 0.0, q), fmt)
            fp8_put_codes(pool, name, blk, off, codes)
            if where == "token":
                fp8t_scales(pool, name)[blk, :, off] = s[..., 0].astype(np.float32)
        return
    if pool.kind == "fp4":
        hkv = pool.num_kv_heads
        for name, rows in (("k", k_rows), ("v", v_rows)):
            x_all = act_decode(np.asarray(rows)[live], act)  # [n, Hkv, D]
            idx_arr = fp4_records(pool, name)
            scale_arr = fp4_scales(pool, name)
            slot0_arr, val_arr = fp4_slot0(pool, name), A[name + "_out_val"]
            # step 1-2: calibrate blocks this call opens, on this call's tokens
            side = 0 if name == "k" else 1
            for b in np.unique(blk):
                rows_in_b = np.nonzero(blk == b)[0]
                for h in range(hkv):
                    if idx_arr[b, h, 0] != UNCALIBRATED:
                        continue
                    if seq_records is not None:
                        lead = rows_in_b[np.argmin(off[rows_in_b])]
                        sq = int(np.asarray(token_seq)[live[lead]])
                        rec = np.asarray(seq_records)[sq, side, h].copy()
                        rec[1 + rec[0]:] = UNCALIBRATED
                        idx_arr[b, h, :] = rec
                        continue
                    o = fp4_calibrate(x_all[rows_in_b, h, :])
                    if calib_log is not None:
                        calib_log.append((name, int(b), h,
                                          fp4_calibration_margin(x_all[rows_in_b, h, :])))
                    rec = np.full(16, UNCALIBRATED, dtype=np.uint8)
                    rec[0] = len(o)
                    rec[1:1 + len(o)] = o
                    idx_arr[b, h, :] = rec
            # step 3: encode every row with its block's channel set
            for i in range(len(live)):
                for h in range(hkv):
                    rec = idx_arr[blk[i], h]
                    o = rec[1:1 + rec[0]].astype(np.int64)
                    packed, s, ov = fp4_encode_row(x_all[i, h, :], o)
                    codes = np.empty(2 * len(packed), dtype=np.uint8)
                    codes[0::2], codes[1::2] = packed & 0xF, packed >> 4
                    fp4_put_codes(pool, name, blk[i], h, off[i], codes)
                    scale_arr[blk[i], h, off[i]] = s
                    if len(o):
                        slot0_arr[blk[i], h, off[i]] = ov[0]
                        val_arr[blk[i], h, :len(o) - 1, off[i]] = ov[1:]
        return
    raise ValueError(pool.kind)


# ----------------------------------------------------------------------------------
# dequantization and gather
# ----------------------------------------------------------------------------------


def dequant_slot_rows(pool: Pool, blk, off, k_scale=None, v_scale=None):
    """Dequantized K and V rows [n, Hkv, D] (fp64, exact) at (blk[i], off[i])."""
    A = pool.arrays
    blk = np.asarray(blk, dtype=np.int64)
    off = np.asarray(off, dtype=np.int64)
    out = []
    for name, sc in (("k", k_scale), ("v", v_scale)):
        if pool.kind == "bf16":
            out.append(act_decode(A[name][blk, :, off, :], "bf16"))
        elif pool.kind == "f16":
            out.append(f16_decode(A[name][blk, :, off, :]))
        elif pool.kind in FP8_KINDS:
            fmt, where = FP8_KINDS[pool.kind]
            if where == "head":
                s = np.asarray(sc, dtype=np.float32).astype(np.float64)[None, :, None]
            else:
                s = fp8t_scales(pool, name)[blk, :, off].astype(np.float64)[..., None]
            out.append(fp8_decode(fp8_get_codes(pool, name, blk, off), fmt) * s)
        elif pool.kind == "fp4":
            codes = fp4_get_codes(pool, name)[blk, :, off, :]  # [n, Hkv, D]
            n, hkv = codes.shape[:2]
            s = fp4_scales(pool, name)[blk, :, off].astype(np.float64)[..., None]
            x = e2m1_decode(codes) * s
            rec = fp4_records(pool, name)[blk]  # [n, Hkv, 16]
            for i in range(n):
                for h in range(hkv):
                    cnt = int(rec[i, h, 0])
                    assert cnt != UNCALIBRATED, "read of a block that was never written"
                    if cnt == 0:
                        continue
                    vals = fp4_outlier_values(pool, name, blk[i], h)  # [CAP, 16]
                    for j in range(cnt):
                        x[i, h, rec[i, h, 1 + j]] = f16_decode(vals[j, off[i]])
            out.append(x)
        else:
            raise ValueError(pool.kind)
    return out[0], out[1]


def gather_sequence(pool: Pool, block_table_row, context_len, k_scale=None, v_scale=None):
    """K̂, V̂ [L, Hkv, D] of one sequence: token t lives at
    (block_table_row[t // 16], t % 16)."""
    t = np.arange(int(context_len))
    blk = np.asarray(block_table_row, dtype=np.int64)[t // BLOCK_TOKENS]
    assert (blk >= 0).all() and (blk < pool.num_blocks).all()
    return dequant_slot_rows(pool, blk, t % BLOCK_TOKENS, k_scale, v_scale)


__all__ = [
    "BLOCK_TOKENS", "OUTLIER_SIGMAS", "UNCALIBRATED", "Pool", "outlier_capacity",
    "fp4_tile_bytes", "fp4_code_map", "fp4_code_bytes", "fp4_get_codes", "fp4_put_codes",
    "fp4_scales", "fp4_records", "fp4_slot0",
    "fp4_outlier_values",
    "FP8_KINDS", "fp8t_run_bytes", "fp8t_codes", "fp8t_scales", "fp8_token_scale",
    "fp8_v_byte", "fp8_put_codes", "fp8_get_codes",
    "fp8_head_scale", "fp4_calibrate", "fp4_calibration_margin", "fp4_encode_row",
    "cache_write", "dequant_slot_rows", "gather_sequence", "f32_round",
]
