// pa_encode.h - the FP8 encoder of the cache write, shared by the write kernels and the
// decode that appends each sequence's new token itself (internal to libpa).
#pragma once

#include "pa_device.h"

namespace pa {

// FP8 (E4M3 or E5M2), 16 values per thread: code = FP8(fp32(x / s)), with the fp32 quotient
// correctly rounded; s is the kv head's scale, or the row's own (per-token pools).
//
// The quotient x / |s| comes from y = fp32(1 / |s|) (correctly rounded, once per thread)
// and two correction steps: q <- q - (|s| q - x) y, each remainder |s| q - x formed by one
// fma; a negative scale then flips the codes' sign bits (the encoding is symmetric).
// Starting from q = fp32(x y), within 2 ulps of x / s, the first step lands within one
// ulp, and from there one step with a correctly rounded reciprocal gives the correctly
// rounded quotient (Markstein's theorem on fma-based division), so the fast form is
// exact, not a guess with a fallback. It needs no overflow and no underflow of the
// remainder where the code is decided: x is first clamped to +-fp32(B |s|), B = 440
// (E4M3) or 56000 (E5M2), past the last rounding midpoint below the largest value (432,
// 53248), so any larger |x / s| saturates either way and the clamped quotient stays inside
// the format's range, and 2^-80 <= |s| <= 2^100 keeps every remainder of a quotient
// above 2^-20 exact (smaller quotients encode as a signed zero, and the steps keep the
// quotient's sign, that of zero included, as y > 0). Other scales, and NaN inputs, take
// the IEEE division and the software encoder.
//
// gfx950's fp32 -> FP8 conversions (v_cvt_pk_fp8_f32 for E4M3, v_cvt_pk_bf8_f32 for E5M2:
// nearest, ties to even) give the same byte as the software encoders for every non-NaN
// fp32 input inside the format's range.
template <bool BF16>
__device__ __forceinline__ uint32_t act_nan_pair(uint32_t u) {
  // nonzero when a 16-bit half is a NaN: |bits| above the infinity pattern (0x7F80 bf16,
  // 0x7C00 fp16) carries into bit 15
  return ((u & 0x7FFF7FFFu) + (BF16 ? 0x007F007Fu : 0x03FF03FFu)) & 0x80008000u;
}

template <bool BF16, bool E5>
__device__ __forceinline__ uint4 fp8_encode16(const uint4 lo, const uint4 hi, float s, bool fast) {
  const float sa = __builtin_fabsf(s);
  const float y = 1.0f / sa, bound = (E5 ? 56000.0f : 440.0f) * sa;
  const uint32_t flip = s < 0.0f ? 0x80808080u : 0u;
  const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  float x[16], q[16];
  uint32_t nan = 0u;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    x[e] = act_to_f32<BF16>((w[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
    const float xc = __builtin_amdgcn_fmed3f(x[e], -bound, bound);
    float t = xc * y;
    float r = __builtin_fmaf(sa, t, -xc);
    t = __builtin_fmaf(-r, y, t);
    r = __builtin_fmaf(sa, t, -xc);
    q[e] = __builtin_fmaf(-r, y, t);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) nan |= act_nan_pair<BF16>(w[i]);
  // byte j of the result holds value j
  uint32_t out[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (E5) {
      out[i] = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(q[4 * i], q[4 * i + 1], 0, false);
      out[i] = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(q[4 * i + 2], q[4 * i + 3],
                                                         (int)out[i], true) ^ flip;
    } else {
      out[i] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[4 * i], q[4 * i + 1], 0, false);
      out[i] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[4 * i + 2], q[4 * i + 3],
                                                         (int)out[i], true) ^ flip;
    }
  }
  if (!fast || nan != 0u) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[i] = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float t = x[4 * i + j] / s;
        out[i] |= (E5 ? encode_e5m2(t) : encode_e4m3(t)) << (8 * j);
      }
    }
  }
  if (s == 0.0f) out[0] = out[1] = out[2] = out[3] = 0u;  // a zero scale stores zero codes
  return make_uint4(out[0], out[1], out[2], out[3]);
}

}  // namespace pa
