// pa_prefill.hip - multi-token paged attention on gfx950, every pool format: the
// queries of a prompt chunk processed after their keys and values were written (chunked
// prefill, dailyaiworld.com, "vLLM 0.7 Ships Unified KV Cache Compression", engine diagram
// with 512-token chunks), or the tokens a draft model proposed (inferensys glossary
// "vLLM", speculative decoding entry). Query i of a sequence with n queries and context L
// sits at position L - n + i and attends causally to positions 0 .. L - n + i.
//
// Work decomposition
//   grid (query tile x kv head, sequence), 4 waves per workgroup. A wave owns NCT tiles of
//   16 MFMA columns; a column is one (query, head) pair, the G heads of a query side by
//   side, so a wave takes 16 NCT / G consecutive queries. It walks the sequence's blocks
//   two at a time, up to its last query's position, and every tile it loads and converts
//   feeds all NCT column tiles.
//
// Per pair of 16-token blocks A, B (lane l: c = l % 16, kg = l / 16):
//   S^T = K Q^T   one 16x16x32 MFMA per 32 channels, block and column tile; lane (c, kg)
//                 then holds column c's logits of tokens 4 kg .. 4 kg + 3 of A and of B;
//   softmax       per column, base 2, running max and sum, lazy rescale, causal limits
//                 per column (blocks wholly before the wave's first query need none);
//   O^T += V^T P^T one 16x16x32 MFMA per 16 output channels and column tile, the k index
//                 running over the 32 tokens of the pair: k = 8 kg + i holds token
//                 4 kg + i of A (i < 4) or 4 kg + i - 4 of B (i >= 4) - the order in which
//                 the lane already holds both its probabilities and its V^T values. P
//                 enters as a hi + lo pair of 16-bit values (about 16 significant bits in bf16,
//                 22 in fp16).
// FP4 pools (dailyaiworld.com, same page, "Technical Breakdown", step 4): the logits take
// the token scale and the K outliers' fp16 terms (q from the fragments already in LDS), P
// takes the V token scale, and each V outlier's term goes straight into the accumulator
// register of its channel (register indexing with a wave-uniform channel).
#include <type_traits>

#include "pa_device.h"
#include "pa_launch.h"
#include "pa_tile.h"

namespace pa {
namespace {

constexpr int kWaves = 4;

// An FP4 outlier record in scalar registers: the count (capped) and the channel bytes
// 1 .. 11 of the record's first three words
struct Rec {
  uint32_t w[3];
  int n;
  __device__ int channel(int j) const {
    const int pos = 1 + j;
    return (int)((w[pos >> 2] >> ((pos & 3) * 8)) & 0xFFu);
  }
};
constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold, log2 units

// q fragments of one wave in LDS: [NCT][KS][64 lanes] x 16 bytes
template <int D, int NCT>
constexpr int q_lds_bytes() { return NCT * (D / 32) * 64 * 16; }

// at least 2 waves per SIMD (256 registers per lane)
template <int KV, int D, bool QBF, int NCT>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2)))
void k_prefill_mt(DecodeArgs a) {
  using G_ = Geo<KV, D>;
  constexpr int KS = G_::KS, NT = G_::NT, DL = G_::DL;
  // PV MFMA type: bf16 for bf16 pools and where P takes the V token scale (FP4, per-token
  // FP8: p s_t may leave fp16's range), else fp16 (E4M3 and E5M2 codes are fp16 values, and
  // P's hi + lo pair then carries 22 bits at fewer instructions)
  constexpr bool PVB = KV == KV_BF16 || tok_scaled(KV);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, kg = lane >> 4;
  // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin by linear id, so
  // linear id w runs on XCD w % 8; renumbering it xcd * (its share) + w / 8 gives each
  // XCD a contiguous range of (sequence, query tile) work, and all query tiles of a
  // sequence meet in one XCD's L2, where its K/V (2 MB at 8192 FP8 tokens) stays resident.
  unsigned xw, yw;
  {
    const unsigned X = gridDim.x, N = X * gridDim.y;
    const unsigned w = blockIdx.y * X + blockIdx.x;
    const unsigned per = N / 8, rem = N % 8, xcd = w % 8, k = w / 8;
    const unsigned wr = xcd < rem ? xcd * (per + 1) + k : rem * (per + 1) + (xcd - rem) * per + k;
    xw = wr % X;
    yw = wr / X;
  }
  const int kvh = (int)(xw % (unsigned)a.num_kv_heads);
  const int qt = (int)(xw / (unsigned)a.num_kv_heads);
  const int s = (int)yw;
  const int G = a.group, Hq = a.num_q_heads;
  const int QPW = 16 * NCT / G;  // queries per wave

  const int L = a.context_lens[s];
  const int q0 = a.query_start[s];
  const int nq = a.query_start[s + 1] - q0;
  const int j0 = (qt * kWaves + wave) * QPW;  // first query of this wave
  const bool rows_ok = q0 >= 0 && nq >= 0 && (int64_t)q0 + nq <= a.num_queries;
  if (L < 1 || L > a.max_blocks * kBlock || !rows_ok || nq > L || nq > a.max_query_len) {
    if (lane == 0 && wave == 0 && qt == 0 && kvh == 0 && a.err)
      atomicOr(a.err, PA_DEVERR_BAD_CONTEXT);
    if (rows_ok && nq <= a.max_query_len)  // zero this wave's rows
      for (int j = j0; j < min(j0 + QPW, nq); ++j)
        for (int i = lane; i < G * D; i += 64)
          a.out[((int64_t)(q0 + j) * Hq + kvh * G) * D + i] = 0.0f;
    return;
  }
  if (j0 >= nq) return;  // no query for this wave

  // keys [0, end) cover the wave's last query; blocks below nfull precede its first one
  const int end = L - nq + min(j0 + QPW, nq);
  const int nblk = (end + kBlock - 1) / kBlock;
  const int nfull = (L - nq + j0 + 1) / kBlock;

  // ---- this lane's columns: query jq[ct] (head col % G), keys below col_end[ct] ----
  // The q fragments wait in LDS, each lane reading back only what it wrote (no barrier):
  // registers go to the accumulators of more column tiles instead.
  extern __shared__ uint4 q_lds_all[];
  uint4* const q_wave = q_lds_all + (int64_t)wave * NCT * KS * 64;
  uint4* const q_lds = q_wave + lane;
  int col_end[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int col = 16 * ct + c;
    const int jq = j0 + col / G;
    const bool qok = jq < nq;
    col_end[ct] = qok ? L - nq + jq + 1 : 0;
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q) +
                          (((int64_t)(q0 + (qok ? jq : 0)) * Hq + kvh * G + col % G) * D +
                           DL * kg) * 2;
#pragma unroll
    for (int t = 0; t < KS; ++t)
      q_lds[(ct * KS + t) * 64] =
          qok ? reinterpret_cast<const uint4*>(qrow)[t] : make_uint4(0, 0, 0, 0);
  }
  float cz = a.sm_scale_log2;
  if constexpr (head_scaled(KV)) cz *= a.k_scale[kvh];

  // ---- block ids: 64 per register, read with readlane ----
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks;
  auto load_ids = [&](int chunk) -> int {
    const int x = chunk * 64 + lane;
    return x < nblk ? bt[x] : 0;
  };
  int ids_a = load_ids(0), ids_b = load_ids(1);
  const uint8_t* kpool = reinterpret_cast<const uint8_t*>(a.k);
  const uint8_t* vpool = reinterpret_cast<const uint8_t*>(a.v);
  const int k_lane_off = c * G_::ROWB + kg * G_::KLANEB;
  const int v_lane_off = 4 * kg * G_::ROWB + c * G_::VLANEB;
  int err_bits = 0;

  // block x of the sequence (x < nblk); ids are consumed in order, so the register pair
  // slides by one chunk when x reaches a multiple of 64
  auto load_tile = [&](Tile<KV, D>& T, int x) {
    if (x > 0 && (x & 63) == 0) {
      ids_a = ids_b;
      ids_b = load_ids((x >> 6) + 1);
    }
    const int b_raw = __builtin_amdgcn_readlane(ids_a, x & 63);
    T.jb = x;
    T.ok = (unsigned)b_raw < (unsigned)a.num_blocks;
    err_bits |= T.ok ? 0 : PA_DEVERR_BAD_BLOCK;
    T.tile = (int64_t)(T.ok ? b_raw : 0) * a.num_kv_heads + kvh;
    load_words(T.k, kpool + T.tile * G_::TILEB + k_lane_off);
    if constexpr (KV == KV_FP4) {
      const uint8_t* kt = kpool + T.tile * G_::TILEB;
      const uint8_t* vt = vpool + T.tile * G_::TILEB;
      // V is stored by channel: one chunk, channels NT c .. NT c + NT - 1 of tokens
      // 4 kg .. 4 kg + 3
      fp4_v_chunk<D, false>(T, vt, c, kg);
      // per-token scales, the first word of each outlier record (lanes 0-31 K's, 32-63
      // V's) and the first outlier slot, which a full block usually fills exactly
      T.sk = reinterpret_cast<const float4*>(kt + PA_FP4_SCALE_OFF(D))[kg];
      T.sv = reinterpret_cast<const float4*>(vt + PA_FP4_SCALE_OFF(D))[kg];
      T.r0 = *reinterpret_cast<const uint32_t*>((lane < 32 ? kt : vt) + PA_FP4_RECORD_OFF(D));
      T.k_o0 = reinterpret_cast<const uint2*>(kt + PA_FP4_SLOT0_OFF(D))[kg];
      T.v_o0 = reinterpret_cast<const uint2*>(vt + PA_FP4_SLOT0_OFF(D))[kg];
    } else if constexpr (is_f8(KV)) {
      f8_v_chunk<KV, D, false>(T, vpool + T.tile * G_::VTILEB, c, kg);  // stored by channel
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        load_words(T.v[r], vpool + T.tile * G_::VTILEB + v_lane_off + r * G_::ROWB);
    }
    if constexpr (f8_tok(KV)) {
      T.sk = reinterpret_cast<const float4*>(kpool + T.tile * G_::TILEB + PA_FP8T_SCALE_OFF(D))[kg];
      T.sv = reinterpret_cast<const float4*>(kpool + T.tile * G_::TILEB + PA_FP8T_VSCALE_OFF(D))[kg];
    }
  };
  // the second block of a last, odd pair: no bytes, every token invalid
  auto empty_tile = [&](Tile<KV, D>& T, int x) {
#pragma unroll
    for (int i = 0; i < G_::KW; ++i) T.k[i] = 0u;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < G_::VW; ++i) T.v[r][i] = 0u;
    T.sk = T.sv = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    T.r0 = 0u;  // no outliers
    T.k_o0 = T.v_o0 = make_uint2(0u, 0u);
    T.jb = x;
    T.ok = false;
    T.tile = 0;
  };

  // ---- online softmax state, per column tile ----
  float m[NCT], l[NCT];
  f32x4 acc[NCT][NT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    m[ct] = -INFINITY;
    l[ct] = 0.0f;
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[ct][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  bool started = false;  // wave-uniform

  auto compute = [&](Tile<KV, D>& TA, Tile<KV, D>& TB, auto kFull) {
    constexpr bool FULL = decltype(kFull)::value;
    if constexpr (!FULL && KV != KV_FP4) {
      // V bytes of tokens past the wave's last key are arbitrary (a NaN code times p = 0
      // is still NaN): zeroed, with the wave's bound, which holds for every column (E2M1
      // has no NaN code, so FP4 codes need no zeroing)
      auto mask_v = [&](Tile<KV, D>& T) {
        if constexpr (is_f8(KV)) {  // byte r of every word is token 4 kg + r
          uint32_t keep = 0u;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            keep |= T.ok && T.jb * kBlock + 4 * kg + r < end ? 0xFFu << (8 * r) : 0u;
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < G_::VW; ++i) T.v[r][i] &= keep;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool keep = T.ok && T.jb * kBlock + 4 * kg + r < end;
#pragma unroll
            for (int i = 0; i < G_::VW; ++i) T.v[r][i] = keep ? T.v[r][i] : 0u;
          }
        }
      };
      mask_v(TA);
      mask_v(TB);
    }
    // FP4 outlier record of one block and side (0: K, from lane 0's word; 1: V, lane 32's),
    // decoded once per pair and used by every column tile; wave-uniform
    auto read_rec = [&](const Tile<KV, D>& T, int side) {
      Rec r;
      r.w[0] = (uint32_t)__builtin_amdgcn_readlane((int)T.r0, 32 * side);
      r.w[1] = r.w[2] = 0u;
      int n = (int)(r.w[0] & 0xFFu);
      if (n > 3 && n != 0xFF) {  // more channels than the first word holds (rare)
        const uint4 x = load_uniform16((side ? vpool : kpool) + T.tile * G_::TILEB +
                                       PA_FP4_RECORD_OFF(D));
        r.w[1] = x.y;
        r.w[2] = x.z;
      }
      if (n == 0xFF) {
        err_bits |= T.ok ? PA_DEVERR_UNCALIBRATED : 0;
        n = 0;
      }
      r.n = n > a.cap ? a.cap : n;
      return r;
    };
    Rec rka, rkb, rva, rvb;
    if constexpr (KV == KV_FP4) {
      rka = read_rec(TA, 0);
      rkb = read_rec(TB, 0);
      rva = read_rec(TA, 1);
      rvb = read_rec(TB, 1);
    }
    // FP4 K outliers of one block for column tile ct: ok[r] = sum_j q[ch_j] o_(4 kg + r),ch_j
    // (fp16 values times the query in fp32). The record sits in scalar registers, so ch is
    // wave-uniform; column c's query value of channel ch is read from the q fragments in
    // LDS, where lane (c, ch / DL) stored it (fragment (ch % DL) / 8, element ch % 8).
    auto k_outliers = [&](const Tile<KV, D>& T, const Rec& rk, int ct, float* ok) {
      ok[0] = ok[1] = ok[2] = ok[3] = 0.0f;
      for (int j = 0; j < rk.n; ++j) {
        const int ch = rk.channel(j);
        const uint16_t* qh = reinterpret_cast<const uint16_t*>(
            q_wave + (ct * KS + (ch % DL) / 8) * 64 + c + 16 * (ch / DL));
        const float qv = act_to_f32<QBF>(qh[ch % 8]);
        const uint2 ov = j == 0 ? T.k_o0
                                : *reinterpret_cast<const uint2*>(
                                      a.k_out_val + ((T.tile * (a.cap - 1) + (j - 1)) * kBlock +
                                                     4 * kg));
        ok[0] = __builtin_fmaf(qv, f16_bits_to_f32(ov.x & 0xFFFFu), ok[0]);
        ok[1] = __builtin_fmaf(qv, f16_bits_to_f32(ov.x >> 16), ok[1]);
        ok[2] = __builtin_fmaf(qv, f16_bits_to_f32(ov.y & 0xFFFFu), ok[2]);
        ok[3] = __builtin_fmaf(qv, f16_bits_to_f32(ov.y >> 16), ok[3]);
      }
    };
    // FP4 V outliers of one block for column tile ct: out[c][ch] += sum_t p_t o_t,ch with
    // the unscaled p of the block's tokens 4 kg .. 4 kg + 3 (p4), summed over the four lanes
    // of the column and added straight into the accumulator register of channel ch
    auto v_outliers = [&](const Tile<KV, D>& T, const Rec& rv, int ct, const float* p4) {
      const int tok0 = T.jb * kBlock + 4 * kg;
      for (int j = 0; j < rv.n; ++j) {
        const int ch = rv.channel(j);
        const uint2 ov = j == 0 ? T.v_o0
                                : *reinterpret_cast<const uint2*>(
                                      a.v_out_val + ((T.tile * (a.cap - 1) + (j - 1)) * kBlock +
                                                     4 * kg));
        // slots of tokens past the wave's last key hold arbitrary bits (maybe NaN): masked
        // with the wave's bound; the causal limits of the columns act through p
        const uint32_t oh[4] = {ov.x & 0xFFFFu, ov.x >> 16, ov.y & 0xFFFFu, ov.y >> 16};
        float part = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool keep = FULL || (T.ok && tok0 + r < end);
          part = __builtin_fmaf(p4[r], keep ? f16_bits_to_f32(oh[r]) : 0.0f, part);
        }
        part = group4_sum(part);
        // channel ch is entry ch % DL = NT r + n, in acc[ct][n][r], of the lanes with
        // kg = ch / DL
        add_entry<NT>(acc[ct], ch % DL, kg == ch / DL ? part : 0.0f);
      }
    };
    // logits of tokens 4 kg .. 4 kg + 3 of one block for column tile ct, masked, before
    // the scale cz (z = x cz, applied where p is formed: exp2(fma(x, cz, -m)))
    auto logits = [&](const Tile<KV, D>& T, const Rec& rk, const f32x4& sa, int ct, float* z) {
      const int tok0 = T.jb * kBlock + 4 * kg;
      float sk[4] = {1.0f, 1.0f, 1.0f, 1.0f};
      if constexpr (tok_scaled(KV)) {
        sk[0] = T.sk.x;
        sk[1] = T.sk.y;
        sk[2] = T.sk.z;
        sk[3] = T.sk.w;
      }
      float ok[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (KV == KV_FP4) k_outliers(T, rk, ct, ok);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool valid = FULL || (T.ok && tok0 + r < col_end[ct]);
        // (sk = 1 folds away; an fma with 1 and 0 would not, as it turns -0 into +0)
        const float x = KV == KV_FP4 ? __builtin_fmaf(sa[r], sk[r], ok[r]) : sa[r] * sk[r];
        z[r] = valid ? x : -INFINITY;
      }
    };
    // logits of both blocks for every column tile; each K fragment feeds NCT MFMAs
    f32x4 sacc[2][NCT];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) sacc[b][ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      const uint4 ka = k_fragment<KV, D, QBF>(TA, t);
      const uint4 kb = k_fragment<KV, D, QBF>(TB, t);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const uint4 qf = q_lds[(ct * KS + t) * 64];
        sacc[0][ct] = mfma_k32(ka, qf, sacc[0][ct], QBF);
        sacc[1][ct] = mfma_k32(kb, qf, sacc[1][ct], QBF);
      }
    }
    // V^T fragments of both blocks, converted while the QK MFMAs run (no dependence)
    uint2 vfa[NT], vfb[NT];
    v_fragments<KV, D, PVB>(TA, vfa);
    v_fragments<KV, D, PVB>(TB, vfb);

    // masked logits and this lane's maxima of every column tile, then one wave-uniform
    // decision for a (rare, lazy) rescale of them all. cz > 0, so the largest scaled
    // logit is cz times the largest unscaled one; m is the same in a column's four lanes,
    // so some column's block maximum passes m + kRescaleLog2 exactly when some lane's own
    // logits do, and the maximum over the column's lanes is taken only then.
    float z[NCT][8], xl[NCT];
    bool grow = false;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      logits(TA, rka, sacc[0][ct], ct, z[ct]);
      logits(TB, rkb, sacc[1][ct], ct, z[ct] + 4);
      xl[ct] = fmaxf(fmaxf(fmaxf(z[ct][0], z[ct][1]), fmaxf(z[ct][2], z[ct][3])),
                     fmaxf(fmaxf(z[ct][4], z[ct][5]), fmaxf(z[ct][6], z[ct][7])));
      grow = grow || xl[ct] * cz > m[ct] + kRescaleLog2;
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const float xg = group4_max(xl[ct]);
        const float mb = xg == -INFINITY ? -INFINITY : xg * cz;  // (-inf times cz = 0: NaN)
        const float mn = fmaxf(m[ct], mb);
        if (started) {
          // (-inf - -inf for a column with nothing unmasked yet: its l and acc are 0 and
          // are left alone)
          const float alpha = m[ct] == mn ? 1.0f : __builtin_amdgcn_exp2f(m[ct] - mn);
          l[ct] *= alpha;
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[ct][n] *= alpha;
        }
        m[ct] = mn;
      }
    }
    started = true;

    uint4 ph[NCT], pl[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // (masked logits are -inf and give p = 0; m is -inf only while every logit of the
        // column so far is masked)
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(z[ct][i], cz, -m[ct]));
        const float p = FULL ? e : (z[ct][i] == -INFINITY ? 0.0f : e);
        l[ct] += p;
        pv[i] = p;
      }
      if constexpr (KV == KV_FP4) {  // before p takes the V token scale
        v_outliers(TA, rva, ct, pv);
        v_outliers(TB, rvb, ct, pv + 4);
      }
      if constexpr (tok_scaled(KV)) {
        // PV runs on the codes: p times the V token scale. A masked token's p is 0 and its
        // scale slot may hold any bits (a NaN times 0 is still NaN), so it stays 0.
        const float sv[8] = {TA.sv.x, TA.sv.y, TA.sv.z, TA.sv.w,
                             TB.sv.x, TB.sv.y, TB.sv.z, TB.sv.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) pv[i] = FULL || pv[i] != 0.0f ? pv[i] * sv[i] : 0.0f;
      }
      uint32_t h[4], lo[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        split2(pv[2 * i], pv[2 * i + 1], PVB, h[i], lo[i]);
      }
      ph[ct] = make_uint4(h[0], h[1], h[2], h[3]);
      pl[ct] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }

#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const uint4 vop = make_uint4(vfa[n].x, vfa[n].y, vfb[n].x, vfb[n].y);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        acc[ct][n] = mfma_k32(vop, ph[ct], acc[ct][n], PVB);
        acc[ct][n] = mfma_k32(vop, pl[ct], acc[ct][n], PVB);
      }
    }
  };

  // ---- pairs of blocks: unmasked ones, then the rest (at most two pairs) ----
  Tile<KV, D> ta, tb;
  const int npair = (nblk + 1) / 2;
  auto load_pair = [&](int pi) {
    load_tile(ta, 2 * pi);
    if (2 * pi + 1 < nblk)
      load_tile(tb, 2 * pi + 1);
    else
      empty_tile(tb, 2 * pi + 1);
  };
  load_pair(0);
  int pi = 0;
  // (a pair with a bad block id takes the masked body, which skips that block, as the
  // decode does; so do the pairs after it - only when ids are bad)
  for (; pi + 1 < npair && 2 * pi + 2 <= nfull && ta.ok && tb.ok; ++pi) {
    compute(ta, tb, std::true_type{});
    load_pair(pi + 1);
  }
  for (; pi < npair; ++pi) {
    compute(ta, tb, std::false_type{});
    if (pi + 1 < npair) load_pair(pi + 1);
  }

  // ---- epilogue ----
  if (err_bits != 0 && lane == 0 && a.err) atomicOr(a.err, err_bits);
  const float vscale = head_scaled(KV) ? a.v_scale[kvh] : 1.0f;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int col = 16 * ct + c;
    const int jq = j0 + col / G;
    const float lt = group4_sum(l[ct]);
    if (jq < nq) {
      const float inv = lt > 0.0f ? vscale / lt : 0.0f;  // 0: every block id was bad
      float* dst = a.out + ((int64_t)(q0 + jq) * Hq + kvh * G + col % G) * D;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int n = 0; n < NT; ++n) dst[DL * kg + NT * r + n] = acc[ct][n][r] * inv;
    }
  }
}

template <int KV, int D, bool QBF, int NCT>
int launch_mt(const DecodeArgs& a, hipStream_t st) {
  const int qpw = 16 * NCT / a.group;
  const int per_wg = kWaves * qpw;
  const int tiles = (a.max_query_len + per_wg - 1) / per_wg;
  if (tiles == 0 || a.num_seqs == 0) return PA_OK;
  const dim3 grid((unsigned)((int64_t)tiles * a.num_kv_heads), (unsigned)a.num_seqs, 1);
  const size_t lds = (size_t)kWaves * q_lds_bytes<D, NCT>();
  hipLaunchKernelGGL((k_prefill_mt<KV, D, QBF, NCT>), grid, dim3(64 * kWaves), lds, st, a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

template <int KV, int D, bool QBF>
int launch_kv(const DecodeArgs& a, int nct, hipStream_t st) {
  return nct == 2 ? launch_mt<KV, D, QBF, 2>(a, st) : launch_mt<KV, D, QBF, 3>(a, st);
}

template <int D>
int launch_d(const DecodeArgs& a, int kv, bool qbf, int nct, hipStream_t st) {
  switch (kv) {
    case KV_F16: return launch_kv<KV_F16, D, false>(a, nct, st);
    case KV_BF16: return launch_kv<KV_BF16, D, true>(a, nct, st);
    case KV_FP8:
      return qbf ? launch_kv<KV_FP8, D, true>(a, nct, st) : launch_kv<KV_FP8, D, false>(a, nct, st);
    case KV_BF8:
      return qbf ? launch_kv<KV_BF8, D, true>(a, nct, st) : launch_kv<KV_BF8, D, false>(a, nct, st);
    case KV_FP8T:
      return qbf ? launch_kv<KV_FP8T, D, true>(a, nct, st) : launch_kv<KV_FP8T, D, false>(a, nct, st);
    case KV_BF8T:
      return qbf ? launch_kv<KV_BF8T, D, true>(a, nct, st) : launch_kv<KV_BF8T, D, false>(a, nct, st);
    case KV_FP4:
      return qbf ? launch_kv<KV_FP4, D, true>(a, nct, st) : launch_kv<KV_FP4, D, false>(a, nct, st);
  }
  return PA_ERR_DTYPE;
}

}  // namespace

int launch_prefill(const DecodeArgs& a, int kv, bool qbf, int D, int col_tiles,
                   hipStream_t st) {
  // column tiles per wave: 3, or 2 for FP4 pools, whose tiles carry scales, records and
  // outlier slots (3 spill there: 258 vs 316 TFLOP/s on the long-context workload);
  // col_tiles 2 or 3 overrides (pa_launch_options), for tuning
  const int nct = col_tiles == 2 || col_tiles == 3 ? col_tiles : kv == KV_FP4 ? 2 : 3;
  return D == 128 ? launch_d<128>(a, kv, qbf, nct, st) : launch_d<64>(a, kv, qbf, nct, st);
}

}  // namespace pa
