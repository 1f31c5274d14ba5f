// pa_device.h - device-side building blocks shared by the gfx950 kernels of libpa.
//
// Number formats (the pages name them, the bit layouts are the OCP ones):
//   E4M3FN: bias 7, subnormals m * 2^-9, largest finite 448 (S.1111.110), NaN S.1111.111.
//   E2M1:   bias 1, magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6.
// Encoders round the fp32 value they are given to the nearest code, ties to the even code,
// saturate at the largest finite magnitude and keep the sign of zero.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlock = 16;          // tokens per physical block
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kOutlierSigmas = 3.2f;  // outlier threshold, in standard deviations

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <typename T, typename F>
__device__ __forceinline__ T bitcast(const F& f) {
  static_assert(sizeof(T) == sizeof(F), "bitcast size");
  return __builtin_bit_cast(T, f);
}

// Load 16 bytes that are the same for the whole wave and are not written while the
// kernel runs (an address computed from wave-uniform values): reading them through the
// constant address space makes the compiler use a scalar load into scalar registers.
__device__ __forceinline__ uint4 load_uniform16(const void* p) {
  typedef __attribute__((address_space(4))) const uint32_t cu32;
  cu32* q = (cu32*)(uintptr_t)p;
  return make_uint4(q[0], q[1], q[2], q[3]);
}

// ---------------------------------------------------------------------------------
// 16-bit activations -> fp32 (exact)
// ---------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b16) {
  return (float)bitcast<_Float16>((uint16_t)b16);
}
template <bool BF16>
__device__ __forceinline__ float act_to_f32(uint32_t b16) {
  return BF16 ? bf16_bits_to_f32(b16) : f16_bits_to_f32(b16);
}

// ---------------------------------------------------------------------------------
// Encoders (software, exact; the inputs are already the fp32 values to be encoded)
// ---------------------------------------------------------------------------------

// fp32 -> E4M3FN byte.
__device__ __forceinline__ uint32_t encode_e4m3(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  if (__builtin_isnan(v)) return sign | 0x7Fu;
  const float a = fminf(__builtin_fabsf(v), 448.0f);  // saturate (448 is the largest finite)
  uint32_t code;
  if (a < 0x1p-6f) {
    // subnormal range: value = m * 2^-9, m = a * 512 rounded to nearest even (0..8;
    // 8 is the smallest normal, code 0x08). Scaling by 512 is exact.
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    // normal: round the 23-bit fp32 mantissa to 3 bits (nearest, ties even); a carry
    // moves into the exponent, which is rebiased from 127 to 7.
    uint32_t b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);
    code = (b >> 20) - (120u << 3);
  }
  return sign | code;
}

// fp32 -> E5M2 byte (OCP: bias 15, two mantissa bits, largest finite 57344): nearest, ties
// to even, saturating to +-57344, sign of zero kept, NaN -> S.11111.11.
__device__ __forceinline__ uint32_t encode_e5m2(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  if (__builtin_isnan(v)) return sign | 0x7Fu;
  const float a = fminf(__builtin_fabsf(v), 57344.0f);
  uint32_t code;
  if (a < 0x1p-14f) {
    // subnormal range: value = m * 2^-16, m = a * 65536 rounded to nearest even (0..4;
    // 4 is the smallest normal, code 0x04). Scaling by 65536 is exact.
    code = (uint32_t)__builtin_rintf(a * 65536.0f);
  } else {
    // normal: round the 23-bit fp32 mantissa to 2 bits (nearest, ties even); a carry
    // moves into the exponent, which is rebiased from 127 to 15.
    uint32_t b = __float_as_uint(a);
    b += 0xFFFFFu + ((b >> 21) & 1u);
    code = (b >> 21) - (112u << 2);
  }
  return sign | code;
}

// fp32 -> E2M1 nibble. Thresholds are the midpoints of the grid 0 .5 1 1.5 2 3 4 6; at an
// exact midpoint the comparison (> or >=) sends the value to the even code.
__device__ __forceinline__ uint32_t encode_e2m1(float v) {
  const float a = __builtin_fabsf(v);
  uint32_t code = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
                  (a >= 3.5f) + (a > 5.0f);
  return code | ((__float_as_uint(v) >> 28) & 8u);
}

// ---------------------------------------------------------------------------------
// Wave-level reductions (wave64). Butterflies, so every lane ends with the result.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Combine the four lanes {l, l^16, l^32, l^48}: the four k-groups of one MFMA column.
// gfx950's v_permlane16_swap / v_permlane32_swap exchange 16-lane rows (resp. 32-lane
// halves) between two registers in the vector ALU; swapping a value with itself leaves
// x_l in one result and x_(l^16) (resp. x_(l^32)) in the other, so combining the two
// results is one butterfly step, with no trip through the LDS crossbar.
// The maximum of two values a permlane swap returned. fmaxf would first quiet each
// operand (a v_max of the value with itself), since the compiler cannot tell that the
// swapped bits are already canonical floats; they are (each lane's own VALU result), so
// one v_max_f32 gives fmaxf's answer.
__device__ __forceinline__ float max_of_swapped(uint32_t a, uint32_t b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return max_of_swapped(r[0], r[1]);
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return max_of_swapped(r[0], r[1]);
}
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float group4_max(float x) { return xor32_max(xor16_max(x)); }
__device__ __forceinline__ float group4_sum(float x) { return xor32_sum(xor16_sum(x)); }

// ---------------------------------------------------------------------------------
// MFMA wrappers (16x16 output tiles; lane l holds column l%16, rows 4*(l/16)+r).
// ---------------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma_k32(const uint4& a, const uint4& b, f32x4 c, bool bf16) {
  if (bf16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(a), bitcast<bf16x8>(b), c, 0,
                                                   0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<f16x8>(a), bitcast<f16x8>(b), c, 0, 0,
                                                0);
}
__device__ __forceinline__ f32x4 mfma_k16(const uint2& a, const uint2& b, f32x4 c, bool bf16) {
  if (bf16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bitcast<bf16x4>(a), bitcast<bf16x4>(b), c,
                                                     0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x16f16(bitcast<f16x4>(a), bitcast<f16x4>(b), c, 0, 0, 0);
}

// Two fp32 -> packed 16-bit pair (round to nearest even), low half = x.
__device__ __forceinline__ uint32_t pack2(float x, float y, bool bf16) {
  if (bf16) return bitcast<uint32_t>(bf16x2{(__bf16)x, (__bf16)y});
  return bitcast<uint32_t>(f16x2{(_Float16)x, (_Float16)y});
}
__device__ __forceinline__ float lo16_to_f32(uint32_t w, bool bf16) {
  return bf16 ? bf16_bits_to_f32(w & 0xFFFFu) : f16_bits_to_f32(w & 0xFFFFu);
}
__device__ __forceinline__ float hi16_to_f32(uint32_t w, bool bf16) {
  return bf16 ? __uint_as_float(w & 0xFFFF0000u) : f16_bits_to_f32(w >> 16);
}

// x - h, h the fp16 value in the low (HI = false) or high half of w, in one v_fma_mix_f32
// (the instruction reads the fp16 half itself; written out, the compiler converts the half
// to fp32 first and subtracts after).
template <bool HI>
__device__ __forceinline__ float sub_f16_half(float x, uint32_t w) {
  float r;
  if constexpr (HI)
    asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(x));
  else
    asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(x));
  return r;
}

// A pair of fp32 values as two 16-bit pairs, hi = (x, y) rounded and lo = their remainders
// rounded: hi + lo carries about 16 significant bits in bf16 and 22 in fp16. (A remainder
// x - hi is exact in fp32.)
__device__ __forceinline__ void split2(float x, float y, bool bf16, uint32_t& hi, uint32_t& lo) {
  hi = pack2(x, y, bf16);
  if (bf16)
    lo = pack2(x - lo16_to_f32(hi, true), y - hi16_to_f32(hi, true), true);
  else
    lo = pack2(sub_f16_half<false>(x, hi), sub_f16_half<true>(y, hi), false);
}

}  // namespace pa
