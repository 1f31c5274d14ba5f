"""Number formats of the paged KV cache, written out from their definitions (fp64, CPU).

TEST INFRASTRUCTURE. This package is the plain, slow CPU reference the HIP path is
checked against. Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg
may import it; nothing in the product path does.

Formats used by the pages:
  * FP8 E4M3 KV cache (xonoai.com field report on vLLM v0.7.2, "Deconstructing the
    v0.7.2 Architecture"; inferensys glossary "vLLM", KV cache quantization entry).
    The variant is the OCP "E4M3FN" one: exponent bias 7, subnormals m*2^-9, largest
    finite value 448 (S.1111.110), NaN = S.1111.111, no infinities.
  * FP8 E5M2 KV cache (same report and section: "FP8 (E4M3 and E5M2)"). OCP E5M2:
    exponent bias 15, subnormals m*2^-16, largest finite value 57344 (S.11110.11),
    infinities S.11111.00, NaN S.11111.xx with xx != 0.
  * 4-bit float KV cache (dailyaiworld.com, "vLLM 0.7 Ships Unified KV Cache
    Compression", section "Technical Breakdown: Dynamic Quantization with Outlier
    Retention", step 3). Read as OCP E2M1: bias 1, magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6.
  * fp16 outlier values (same page, step 2, and the engine diagram's "Outlier Buffer
    [FP16 Precision]").

Rounding readings (the pages are silent): round to nearest, ties to the even code;
magnitudes beyond the largest finite value saturate to it; the sign of zero is kept.
Every encoder here takes the value to be encoded as fp64; the callers decide how that
value was formed (see oracle.cache for the fp32 quotient reading).
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------------
# 16-bit activation formats (inputs arrive as raw uint16 bit patterns)
# ----------------------------------------------------------------------------------


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp64. A bf16 value is the upper half of an fp32 word."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f16_decode(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns -> fp64."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def act_decode(bits: np.ndarray, act: str) -> np.ndarray:
    if act == "bf16":
        return bf16_decode(bits)
    if act == "f16":
        return f16_decode(bits)
    raise ValueError(f"unknown activation dtype {act!r}")


def f16_encode(x: np.ndarray) -> np.ndarray:
    """fp64 -> IEEE binary16 bits, round to nearest even (overflow gives +-inf)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def f32_round(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest fp32 value (ties to even), returned as fp64."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def f32_quotient(x: np.ndarray, s) -> np.ndarray:
    """Correctly rounded fp32 quotient x/s for fp32-representable x and s.

    The fp64 quotient is rounded once more to fp32. For operands that are themselves
    fp32 values this double rounding gives the correctly rounded fp32 result, because
    53 >= 2*24 + 2 (the classical bound for +, -, *, / and sqrt)."""
    x = np.asarray(x, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        return f32_round(x / s)


# ----------------------------------------------------------------------------------
# Grid rounding shared by both small-float encoders (a format-agnostic helper)
# ----------------------------------------------------------------------------------


def _nearest_even_index(a: np.ndarray, mags: np.ndarray) -> np.ndarray:
    """Index of the grid point nearest to a (a >= 0, a <= mags[-1]); ties -> even index.

    mags is the strictly increasing list of non-negative magnitudes of a format, indexed
    by the magnitude bits of the code, so an even index is an even mantissa."""
    hi = np.searchsorted(mags, a, side="left")  # first grid point >= a
    hi = np.clip(hi, 0, len(mags) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    pick = np.where(d_lo < d_hi, lo, hi)
    tie = d_lo == d_hi
    pick = np.where(tie, np.where(lo % 2 == 0, lo, hi), pick)
    return pick.astype(np.int64)


# ----------------------------------------------------------------------------------
# OCP FP8 E4M3FN
# ----------------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_magnitudes() -> np.ndarray:
    """Magnitudes of the 127 finite non-negative E4M3FN codes 0x00..0x7E, by code."""
    out = np.empty(127, dtype=np.float64)
    for code in range(127):
        e, m = code >> 3, code & 7
        if e == 0:
            out[code] = m * 2.0 ** -9  # subnormal: (m/8) * 2^(1-7)
        else:
            out[code] = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_E4M3_MAGS = e4m3_magnitudes()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3FN byte codes -> fp64 (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    mag_bits = c & 0x7F
    val = np.where(mag_bits == 0x7F, np.nan, _E4M3_MAGS[np.minimum(mag_bits, 126)])
    return np.where(c & 0x80, -val, val)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """fp64 -> E4M3FN byte codes: nearest, ties to even, saturating to +-448, sign of
    zero kept, NaN -> S.1111.111."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.uint8) << np.uint8(7)
    nan = np.isnan(v)
    a = np.minimum(np.abs(np.where(nan, 0.0, v)), E4M3_MAX)
    idx = _nearest_even_index(a, _E4M3_MAGS).astype(np.uint8)
    idx = np.where(nan, np.uint8(0x7F), idx)
    return (idx | sign).astype(np.uint8)


# ----------------------------------------------------------------------------------
# OCP FP8 E5M2
# ----------------------------------------------------------------------------------

E5M2_MAX = 57344.0


def e5m2_magnitudes() -> np.ndarray:
    """Magnitudes of the 124 finite non-negative E5M2 codes 0x00..0x7B, by code."""
    out = np.empty(124, dtype=np.float64)
    for code in range(124):
        e, m = code >> 2, code & 3
        if e == 0:
            out[code] = m * 2.0 ** -16  # subnormal: (m/4) * 2^(1-15)
        else:
            out[code] = (1.0 + m / 4.0) * 2.0 ** (e - 15)
    return out


_E5M2_MAGS = e5m2_magnitudes()


def e5m2_decode(codes: np.ndarray) -> np.ndarray:
    """E5M2 byte codes -> fp64 (+-inf for S.11111.00, NaN for S.11111.xx, xx != 0)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    mag_bits = c & 0x7F
    val = np.where(mag_bits == 0x7C, np.inf,
                   np.where(mag_bits > 0x7C, np.nan, _E5M2_MAGS[np.minimum(mag_bits, 123)]))
    return np.where(c & 0x80, -val, val)


def e5m2_encode(v: np.ndarray) -> np.ndarray:
    """fp64 -> E5M2 byte codes: nearest, ties to even, saturating to +-57344 (infinities
    included, as for E4M3), sign of zero kept, NaN -> S.11111.11."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.uint8) << np.uint8(7)
    nan = np.isnan(v)
    a = np.minimum(np.abs(np.where(nan, 0.0, v)), E5M2_MAX)
    idx = _nearest_even_index(a, _E5M2_MAGS).astype(np.uint8)
    idx = np.where(nan, np.uint8(0x7F), idx)
    return (idx | sign).astype(np.uint8)


def fp8_encode(v: np.ndarray, fmt: str) -> np.ndarray:
    """fmt "e4m3" or "e5m2"."""
    return e4m3_encode(v) if fmt == "e4m3" else e5m2_encode(v)


def fp8_decode(codes: np.ndarray, fmt: str) -> np.ndarray:
    return e4m3_decode(codes) if fmt == "e4m3" else e5m2_decode(codes)


def fp8_max(fmt: str) -> float:
    return E4M3_MAX if fmt == "e4m3" else E5M2_MAX


# ----------------------------------------------------------------------------------
# OCP FP4 E2M1
# ----------------------------------------------------------------------------------

E2M1_MAX = 6.0


def e2m1_magnitudes() -> np.ndarray:
    """Magnitudes of the 8 non-negative E2M1 codes 0..7 (bias 1, one mantissa bit)."""
    out = np.empty(8, dtype=np.float64)
    for code in range(8):
        e, m = code >> 1, code & 1
        if e == 0:
            out[code] = m * 0.5  # subnormal: (m/2) * 2^(1-1)
        else:
            out[code] = (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return out


_E2M1_MAGS = e2m1_magnitudes()


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """4-bit E2M1 codes (0..15, sign in bit 3) -> fp64."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    val = _E2M1_MAGS[c & 7]
    return np.where(c & 8, -val, val)


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """fp64 -> 4-bit E2M1 codes: nearest, ties to even, saturating to +-6, sign of zero
    kept. Inputs must not be NaN (the format has no NaN)."""
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("E2M1 has no NaN encoding")
    sign = np.signbit(v).astype(np.uint8) << np.uint8(3)
    a = np.minimum(np.abs(v), E2M1_MAX)
    return (_nearest_even_index(a, _E2M1_MAGS).astype(np.uint8) | sign).astype(np.uint8)
