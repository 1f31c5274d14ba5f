"""FP4 calibration variants: attention error against exact attention over the unquantized
inputs, and bytes per token. A study built on the oracle's primitives, run by hand; it is
not part of the parity oracle (its variant quantizers - capacity k, fp16 scales, no
outliers - are measured here, not pinned) and never feeds the product path:

    python tests/studies/fp4_variants.py [--seqs 4] [--tokens 4096] [--decode 64]

Sequences are written as the serving loop writes them: a prompt in 512-token prefill
chunks, then `decode` generated tokens one call each (dailyaiworld.com, "vLLM 0.7 Ships
Unified KV Cache Compression": 512-token chunked prefill, and "Technical Breakdown:
Dynamic Quantization with Outlier Retention", steps 1-4, for the 4-bit scheme). Variants:

  per-block      the kernels' default: a block's outlier set comes from the rows of the
                 first write into it (16 prompt tokens, or 1 generated token)
  per-sequence   one set per (sequence, kv head, K|V) from the first prefill chunk
                 (pa_fp4_sequence_outliers + pa_cache_write_seq_outliers)
  no outliers    plain E2M1 with the per-token scale, no fp16 channels
  capacity k     per-block sets cut to the k channels of largest norm (a smaller outlier
                 buffer: only k fp16 slots per block and head)
  fp16 scales    per-block sets, each token scale rounded to fp16 before encoding
  FP8 E4M3       per-head scale absmax/448 over the sequence (reference point)

Error: decode of 8 query heads per kv head (q ~ N(0,1)) over the dequantized cache
against the same decode over the 16-bit inputs, fp64; relative L2 over all outputs and the
largest absolute difference. Bytes: per token and kv head, K + V, what the pool holds
(footprint) and what a decode reads (a block's runs plus the outlier slots in use).
"""
from __future__ import annotations

import argparse
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from oracle.attention import attend  # noqa: E402
from oracle.cache import fp4_calibrate, fp4_encode_row  # noqa: E402
from oracle.formats import (E2M1_MAX, E4M3_MAX, act_decode, e2m1_decode,  # noqa: E402
                            e2m1_encode, e4m3_decode, e4m3_encode, f16_decode, f16_encode,
                            f32_quotient)

D, HQ, CHUNK, BLOCK = 128, 8, 512, 16
RUN_BYTES = 1152      # codes + token scales + record + first outlier slot, padded to 128
SLOT_BYTES = 32       # one more outlier channel: 16 fp16 values per (block, head, side)
CAP = 11


def _rows(rng, L, planted):
    x = rng.standard_normal((L, D)).astype(np.float32)
    for c, f in planted:
        x[:, c] *= np.float32(f)
    u = x.view(np.uint32)
    bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)  # bf16, nearest even
    return act_decode(bits, "bf16")


def _first_write_rows(L, decode):
    """Rows of the first write into each block: prompt chunks, then one-token calls."""
    prompt = L - decode
    out = []
    for b in range(-(-L // BLOCK)):
        t0 = b * BLOCK
        if t0 < prompt:
            c_end = min((t0 // CHUNK + 1) * CHUNK, prompt)
            out.append(np.arange(t0, min(t0 + BLOCK, c_end)))
        else:
            out.append(np.array([t0]))
    return out


def _largest(x_rows, o, k):
    """The k channels of o with the largest RMS over x_rows, ascending."""
    if len(o) <= k:
        return o
    r = np.sqrt(np.mean(x_rows[:, o] ** 2, axis=0))
    return np.sort(o[np.argsort(-r, kind="stable")[:k]])


def _fp4_dequant(x, sets, scale16=False):
    """Dequantized rows with each block's outlier set (E2M1 inliers, fp16 outliers)."""
    out = np.empty_like(x)
    for t in range(x.shape[0]):
        o = np.asarray(sets[t // BLOCK], dtype=np.int64)
        if not scale16:
            packed, s, ov = fp4_encode_row(x[t], o)
            codes = np.empty(D, dtype=np.uint8)
            codes[0::2], codes[1::2] = packed & 0xF, packed >> 4
            row = e2m1_decode(codes) * np.float64(s)
        else:
            inl = np.ones(D, dtype=bool)
            inl[o] = False
            a = np.abs(x[t, inl]).max() if inl.any() else 0.0
            s = f16_decode(f16_encode(np.asarray(f32_quotient(a, E2M1_MAX))))  # fp16 scale
            row = np.zeros(D)
            if s != 0.0:
                row[inl] = e2m1_decode(e2m1_encode(x[t, inl] / s)) * s
            ov = f16_encode(x[t, o])
        row[o] = f16_decode(ov)
        out[t] = row
    return out


def _fp8_dequant(x):
    s = float(f32_quotient(np.abs(x).max(), E4M3_MAX))
    return e4m3_decode(e4m3_encode(f32_quotient(x, s))) * s


def study(seqs=4, tokens=4096, decode=64, planted=((5, 20.0),), seed=0):
    rng = np.random.default_rng(seed)
    first = _first_write_rows(tokens, decode)
    nblk = len(first)
    names = ["per-block", "per-sequence", "no outliers", "capacity 1", "capacity 2",
             "fp16 scales", "FP8 E4M3"]
    err = {n: [] for n in names}
    ref_all = []
    used = {n: 0 for n in names}  # outlier slots in use, over (block, side)
    for _ in range(seqs):
        x = {side: _rows(rng, tokens, planted) for side in "kv"}
        q = rng.standard_normal((HQ, D))
        deq = {n: {} for n in names}
        for side in "kv":
            xs = x[side]
            blk_sets = [fp4_calibrate(xs[r]) for r in first]
            seq_set = fp4_calibrate(xs[:min(CHUNK, tokens - decode)])
            variants = {
                "per-block": blk_sets,
                "per-sequence": [seq_set] * nblk,
                "no outliers": [np.zeros(0, dtype=np.int64)] * nblk,
                "capacity 1": [_largest(xs[r], o, 1) for r, o in zip(first, blk_sets)],
                "capacity 2": [_largest(xs[r], o, 2) for r, o in zip(first, blk_sets)],
                "fp16 scales": blk_sets,
            }
            for n, sets in variants.items():
                deq[n][side] = _fp4_dequant(xs, sets, scale16=(n == "fp16 scales"))
                used[n] += sum(len(o) for o in sets)
            deq["FP8 E4M3"][side] = _fp8_dequant(xs)
        sm = 1.0 / np.sqrt(D)
        ref = np.stack([attend(q[h], x["k"], x["v"], sm)[0] for h in range(HQ)])
        ref_all.append(ref)
        for n in names:
            got = np.stack([attend(q[h], deq[n]["k"], deq[n]["v"], sm)[0] for h in range(HQ)])
            err[n].append(got - ref)
    ref = np.concatenate(ref_all)
    rows = []
    for n in names:
        e = np.concatenate(err[n])
        rel = float(np.linalg.norm(e) / np.linalg.norm(ref))
        per_side = used[n] / (seqs * 2 * nblk)  # mean outliers per (block, side)
        if n == "FP8 E4M3":
            foot = read = 256.0
        else:
            cap = {"capacity 1": 1, "capacity 2": 2, "no outliers": 0}.get(n, CAP)
            foot = 2 * (RUN_BYTES + SLOT_BYTES * max(cap - 1, 0)) / BLOCK
            read = 2 * (RUN_BYTES + SLOT_BYTES * max(per_side - 1, 0)) / BLOCK
        rows.append((n, rel, float(np.abs(e).max()), per_side, foot, read))
    return rows


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--seqs", type=int, default=4)
    ap.add_argument("--tokens", type=int, default=4096)
    ap.add_argument("--decode", type=int, default=64)
    args = ap.parse_args()
    cases = {
        "one planted channel x20 (the long-context workload's inputs)": ((5, 20.0),),
        "three planted channels x20, x8, x4": ((5, 20.0), (40, 8.0), (77, 4.0)),
    }
    for title, planted in cases.items():
        print(f"\n{title}: {args.seqs} sequences x {args.tokens} tokens "
              f"({args.decode} generated), head_dim {D}, {HQ} query heads")
        print("| variant | rel L2 error | max abs error | outliers per block | footprint B/token | "
              "decode reads B/token |")
        print("|---|---|---|---|---|---|")
        for n, rel, mx, per, foot, read in study(args.seqs, args.tokens, args.decode, planted):
            print(f"| {n} | {rel:.3e} | {mx:.3e} | {per:.2f} | {foot:.1f} | {read:.1f} |")


if __name__ == "__main__":
    main()
