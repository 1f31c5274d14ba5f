// pa_tile.h - the paged K/V tile as the attention kernels read it on gfx950: pool formats,
// per-lane tile geometry, the 16-byte loads of one (block, kv head) tile and the exact
// conversions of its codes into the 16-bit MFMA operands (internal to libpa).
//
// Lane l of a wave (c = l % 16, kg = l / 16) holds, of a 16-token block:
//   K  token c's channels [D/4 kg, D/4 (kg + 1)) - the A operand of S^T = K Q^T, one
//      16x16x32 MFMA per 32 channels (k_fragment);
//   V  tokens 4 kg .. 4 kg + 3 of channels NT c .. NT c + NT - 1 - the A operand of
//      O^T += V^T P^T (v_fragments). 4- and 8-bit V runs store those values by channel (a
//      channel's four tokens together), in the order the lanes load them; 16-bit V runs
//      store token rows, transposed in registers.
#pragma once

#include "../../include/pa.h"
#include "pa_device.h"

namespace pa {

// pool formats (the pa_kv_dtype values)
enum { KV_F16 = 0, KV_BF16 = 1, KV_FP8 = 2, KV_FP4 = 3, KV_BF8 = 4, KV_FP8T = 5, KV_BF8T = 6 };
constexpr bool is_f8(int kv) { return kv == KV_FP8 || kv == KV_BF8 || kv == KV_FP8T || kv == KV_BF8T; }
constexpr bool f8_e5(int kv) { return kv == KV_BF8 || kv == KV_BF8T; }        // E5M2 codes
constexpr bool f8_tok(int kv) { return kv == KV_FP8T || kv == KV_BF8T; }      // per-token scales
constexpr bool head_scaled(int kv) { return kv == KV_FP8 || kv == KV_BF8; }  // per-head scales
constexpr bool tok_scaled(int kv) { return kv == KV_FP4 || f8_tok(kv); }

template <int KV, int D>
struct Geo {
  static constexpr int KS = D / 32;  // QK MFMA steps (k = 32 channels each)
  static constexpr int NT = D / 16;  // PV MFMA tiles (16 output channels each)
  static constexpr int DL = D / 4;   // channels per lane in K fragments and outputs
  static constexpr int EBITS = is_f8(KV) ? 8 : KV == KV_FP4 ? 4 : 16;
  static constexpr int ROWB = D * EBITS / 8;       // bytes of one token row
  // bytes between consecutive (block, head) tiles of the k array (TILEB) and of the v
  // array (VTILEB); an FP4 tile also holds its per-token scales, its outlier record and its
  // first outlier slot after the codes; a per-token FP8 K tile holds the token scales of
  // both K and V after its codes, and its V tile only codes
  static constexpr int TILEB = KV == KV_FP4   ? PA_FP4_TILE_BYTES(D)
                               : f8_tok(KV) ? PA_FP8T_TILE_BYTES(D)
                                            : kBlock * ROWB;
  static constexpr int VTILEB = f8_tok(KV) ? PA_FP8T_VTILE_BYTES(D) : TILEB;
  static constexpr int KW = DL * EBITS / 32;       // K words per lane
  // V words per lane per token; FP4 V is read by channel instead (fp4_v_chunk): T.v[w][0]
  // holds word w of the lane's chunk
  static constexpr int VW = KV == KV_FP4 ? 1 : NT * EBITS / 32;
  static constexpr int KLANEB = DL * EBITS / 8;    // K bytes per lane
  static constexpr int VLANEB = NT * EBITS / 8;    // V bytes per lane per token
};

// N 32-bit words from p (16-byte aligned for N % 4 == 0). NT selects the non-temporal
// form (the loads carry the streaming hint, so the lines they fill are the first the caches
// give up): for K/V tiles that a launch reads exactly once, as in the decode of 8- and
// 4-bit pools (measured on the 70B one-GPU share, FP8, 539 MB per launch: 94.1 -> 89.7 us
// per decode launch). Loops that re-read tiles out of L2 (multi-token queries) keep the
// default form.
template <int N, bool NT = false>
__device__ __forceinline__ void load_words(uint32_t (&w)[N], const uint8_t* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const u32x4* q = reinterpret_cast<const u32x4*>(p) + i;
      const u32x4 x = NT ? __builtin_nontemporal_load(q) : *q;
      w[4 * i] = x.x;
      w[4 * i + 1] = x.y;
      w[4 * i + 2] = x.z;
      w[4 * i + 3] = x.w;
    }
  } else if constexpr (N == 2) {
    const u32x2* q = reinterpret_cast<const u32x2*>(p);
    const u32x2 x = NT ? __builtin_nontemporal_load(q) : *q;
    w[0] = x.x;
    w[1] = x.y;
  } else {
    static_assert(N == 1, "word count");
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
    w[0] = NT ? __builtin_nontemporal_load(q) : *q;
  }
}

// Hardware conversions (scale 1.0, so exact: every E4M3 and E2M1 value is a bf16 and an
// fp16 value). SEL picks the 16-bit half (FP8) or the byte (FP4) of the source word.
template <bool BF, int SEL, bool E5 = false>
__device__ __forceinline__ uint32_t cvt_fp8x2(uint32_t w) {
  if constexpr (E5) {  // E5M2 ("bf8")
    if constexpr (BF)
      return bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, SEL != 0));
    else
      return bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, SEL != 0));
  } else if constexpr (BF) {
    return bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, SEL != 0));
  } else {
    return bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, SEL != 0));
  }
}
template <bool BF, int SEL>
__device__ __forceinline__ uint32_t cvt_fp4x2(uint32_t w) {
  if constexpr (BF)
    return bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL));
  else
    return bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL));
}

template <int KV, int D>
struct Tile {
  using G_ = Geo<KV, D>;
  uint32_t k[G_::KW];
  uint32_t v[4][G_::VW];  // 16-bit: token rows 4 kg .. 4 kg + 3; 8- and 4-bit: the words
                          // of the lane's channel chunk, in order (v[w / VW][w % VW])
  float4 sk, sv;  // FP4 per-token scales of tokens 4 kg .. 4 kg + 3
  uint32_t r0;    // FP4: first word of the K (lanes 0-31) and V (lanes 32-63) records
  uint2 k_o0, v_o0;  // FP4 outlier slot 0 of tokens 4 kg .. 4 kg + 3 (fp16), fetched with
                     // the tile since a full block usually holds exactly one outlier
  int64_t tile;   // b * Hkv + kv head
  int jb;         // logical block index in the sequence
  bool ok;        // block id in range
  bool fresh = false;  // decode with append: the tile whose row this wave wrote in this launch
};

// FP4 V codes of one lane: chunk c * 4 + kg of the tile's first 8 D bytes holds channels
// NT c .. NT c + NT - 1 of tokens 4 kg .. 4 kg + 3 (2 NT bytes: 16 at head_dim 128, 8 at 64),
// loaded with one streaming or ordinary load into T.v[0..NT/2)[0].
template <int D, bool NT_HINT>
__device__ __forceinline__ void fp4_v_chunk(Tile<KV_FP4, D>& T, const uint8_t* tile, int c,
                                            int kg) {
  constexpr int W = D / 32;  // words per chunk
  uint32_t x[W];
  load_words<W, NT_HINT>(x, tile + (c * 4 + kg) * (4 * W));
#pragma unroll
  for (int w = 0; w < W; ++w) T.v[w][0] = x[w];
}

// FP8 V runs (every 8-bit format) are stored by channel, in the order the lanes read them:
// with NT = D / 16, lane (c, kg) needs channels NT c .. NT c + NT - 1 of tokens
// 4 kg .. 4 kg + 3, a 32-bit word per channel (its four token bytes). Those NT words are
// D / 64 pieces of 4 words; piece p of every lane forms 1024 bytes at p * 1024, lane
// l = 16 kg + c at 16 l. So each 16-byte load instruction of the wave reads 1024
// contiguous bytes, whole cache lines (a chunk per lane read in two pieces 16 bytes apart
// would touch every line of the run twice, and the streaming hint can evict a line
// between the two). Token t, channel ch: (j / 4) * 1024 + (16 (t / 4) + ch / NT) * 16 +
// (j % 4) * 4 + t % 4, j = ch % NT. Word w of the lane's channels goes to
// T.v[w / VW][w % VW].
template <int KV, int D, bool NT_HINT>
__device__ __forceinline__ void f8_v_chunk(Tile<KV, D>& T, const uint8_t* run, int c, int kg) {
  constexpr int NT = D / 16, VW = Geo<KV, D>::VW;
  static_assert(4 * VW == NT && NT % 4 == 0, "a lane's pieces fill the tile's V words");
  const uint8_t* at = run + 16u * (16u * (uint32_t)kg + (uint32_t)c);
#pragma unroll
  for (int p = 0; p < NT / 4; ++p) {
    uint32_t x[4];
    load_words<4, NT_HINT>(x, at + 1024 * p);
#pragma unroll
    for (int i = 0; i < 4; ++i) T.v[(4 * p + i) / VW][(4 * p + i) % VW] = x[i];
  }
}
// Store the 16 codes of channels 16 j .. 16 j + 15 of token t (byte e of `codes` is channel
// 16 j + e) into an FP8 V run: one byte per channel.
template <int D>
__device__ __forceinline__ void f8_v_store16(uint8_t* run, int t, int j, const uint4& codes) {
  constexpr int NT = D / 16;
  const uint32_t w[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int ch = 16 * j + e, g = ch / NT, jj = ch % NT;
    run[(jj / 4) * 1024 + (16 * (t / 4) + g) * 16 + (jj % 4) * 4 + t % 4] =
        (uint8_t)(w[e >> 2] >> ((e & 3) * 8));
  }
}

// 16-bit K fragment for step t: 8 values of channels D/4 kg + 8 t + (0..7).
template <int KV, int D, bool QBF>
__device__ __forceinline__ uint4 k_fragment(const Tile<KV, D>& T, int t) {
  if constexpr (KV == KV_F16 || KV == KV_BF16) {
    return make_uint4(T.k[4 * t], T.k[4 * t + 1], T.k[4 * t + 2], T.k[4 * t + 3]);
  } else if constexpr (is_f8(KV)) {
    constexpr bool E5 = f8_e5(KV);
    const uint32_t a = T.k[2 * t], b = T.k[2 * t + 1];
    return make_uint4(cvt_fp8x2<QBF, 0, E5>(a), cvt_fp8x2<QBF, 1, E5>(a),
                      cvt_fp8x2<QBF, 0, E5>(b), cvt_fp8x2<QBF, 1, E5>(b));
  } else {
    const uint32_t a = T.k[t];
    return make_uint4(cvt_fp4x2<QBF, 0>(a), cvt_fp4x2<QBF, 1>(a), cvt_fp4x2<QBF, 2>(a),
                      cvt_fp4x2<QBF, 3>(a));
  }
}

// V^T fragments: vf[n] = channel NT c + n of tokens 4 kg .. 4 kg + 3 as four 16-bit values
// (tokens 0,1 in the low word, 2,3 in the high word).
template <int KV, int D, bool PVB>
__device__ __forceinline__ void v_fragments(const Tile<KV, D>& T, uint2 (&vf)[Geo<KV, D>::NT]) {
  constexpr int NT = Geo<KV, D>::NT;
  if constexpr (KV == KV_FP4) {
    // V is stored by channel: word w of the lane's chunk holds channels 2w, 2w+1, each as
    // two bytes of token pairs (4 kg, 4 kg + 1) and (4 kg + 2, 4 kg + 3); one conversion
    // per byte gives a fragment half directly
#pragma unroll
    for (int w = 0; w < NT / 2; ++w) {
      vf[2 * w].x = cvt_fp4x2<true, 0>(T.v[w][0]);
      vf[2 * w].y = cvt_fp4x2<true, 1>(T.v[w][0]);
      vf[2 * w + 1].x = cvt_fp4x2<true, 2>(T.v[w][0]);
      vf[2 * w + 1].y = cvt_fp4x2<true, 3>(T.v[w][0]);
    }
  } else if constexpr (KV == KV_F16 || KV == KV_BF16) {
    // pairs[r][i] = 16-bit channels (2i, 2i+1) of token r
    uint32_t pairs[4][NT / 2];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int i = 0; i < NT / 2; ++i) pairs[r][i] = T.v[r][i];
    }
#pragma unroll
    for (int i = 0; i < NT / 2; ++i) {
      vf[2 * i].x = __builtin_amdgcn_perm(pairs[1][i], pairs[0][i], 0x05040100u);
      vf[2 * i].y = __builtin_amdgcn_perm(pairs[3][i], pairs[2][i], 0x05040100u);
      vf[2 * i + 1].x = __builtin_amdgcn_perm(pairs[1][i], pairs[0][i], 0x07060302u);
      vf[2 * i + 1].y = __builtin_amdgcn_perm(pairs[3][i], pairs[2][i], 0x07060302u);
    }
  } else {
    // FP8: the lane's chunk holds channel NT c + n of its four tokens in word n; one
    // conversion per token pair
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const uint32_t w = T.v[n / Geo<KV, D>::VW][n % Geo<KV, D>::VW];
      vf[n].x = cvt_fp8x2<PVB, 0, f8_e5(KV)>(w);
      vf[n].y = cvt_fp8x2<PVB, 1, f8_e5(KV)>(w);
    }
  }
}

// acc[n][r] += x for the entry e = NT r + n (wave-uniform) of a lane's output channels
// (channel DL kg + NT r + n of the lane's column, DL = 4 NT). The accumulators are viewed as
// one register vector, so the uniform index becomes the hardware's register indexing
// (s_set_gpr_idx_on) on the registers in place: no copy of the accumulators and no trip
// through memory. (A branch tree over the entries instead is merged by the compiler into
// an indexed store, which moves the accumulators to scratch.)
template <int NT>
__device__ __forceinline__ void add_entry(f32x4 (&acc)[NT], int e, float x) {
  typedef float flat_t __attribute__((ext_vector_type(4 * NT)));
  flat_t w;
#pragma unroll
  for (int t = 0; t < 4 * NT; ++t) w[t] = acc[t / 4][t % 4];
  w[__builtin_amdgcn_readfirstlane(4 * (e % NT) + e / NT)] += x;  // acc[n][r] at 4 n + r
#pragma unroll
  for (int t = 0; t < 4 * NT; ++t) acc[t / 4][t % 4] = w[t];
}

}  // namespace pa
