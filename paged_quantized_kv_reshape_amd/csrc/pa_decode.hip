// pa_decode.hip - paged decode attention for gfx950 (MI355X).
//
// One query token per sequence attends to the K/V of its context, which sits in fixed
// 16-token physical blocks reached through the sequence's block table (inferensys
// glossary "vLLM", PagedAttention entry; xonoai.com field report on vLLM v0.7.2,
// "Deconstructing the v0.7.2 Architecture"). The cache is read as stored: 16-bit values,
// FP8 E4M3 codes times a per-head scale, or E2M1 codes times a per-token scale with the
// block's fp16 outlier channels added back in (dailyaiworld.com, "vLLM 0.7 Ships Unified
// KV Cache Compression", "Technical Breakdown: Dynamic Quantization with Outlier
// Retention", step 4). Long contexts split into partitions that run as independent
// workgroups and are recombined by a log-sum-exp merge (split-KV "Flash-Decoding", the
// same page and its cited sources).
//
// Work decomposition
//   grid (partition, kv head, sequence); a workgroup of W waves covers one partition and
//   wave w takes the partition's blocks w, w + W, w + 2W, ...; the waves' (max, sum, acc)
//   states are merged in LDS at the end. All query heads of a kv head (the GQA group,
//   G <= 16) are processed together by every wave, so each K/V tile is read exactly once.
//
// Per 16-token block, one wave (lane l: c = l % 16, kg = l / 16):
//   S^T = K Q^T   MFMA 16x16x32 (rows = the block's 16 tokens, columns = query heads):
//                 lane (c, kg) loads token c's channels [D/4 kg, D/4 (kg+1)) with 16-byte
//                 loads and holds, after the MFMA, the logits of head c for tokens
//                 4 kg .. 4 kg + 3;
//   softmax       running max m and sum l per head, base 2 (log2 e folded into the
//                 scale); the max over the 4 lanes of a head is a 2-step butterfly; the
//                 accumulator is rescaled only when some head's max grows by more than
//                 kRescale (then every probability stays below 2^kRescale);
//   O^T += V^T P^T MFMA 16x16x16 per 16 output channels (rows = channels, k = tokens):
//                 the probabilities are already in the B-operand layout (head c, tokens
//                 4 kg..4 kg+3); lane (c, kg) loads channels [NT c, NT (c+1)) of tokens
//                 4 kg..4 kg+3 (8- and 4-bit runs store that chunk by channel; 16-bit
//                 token rows are transposed in registers with v_perm) so one register pair
//                 holds one channel of four tokens. P enters as a hi + lo pair of 16-bit
//                 values (about 16 significant bits in bf16, 22 in fp16), so PV loses
//                 nothing to 16-bit rounding of P. After the block loop lane (c, kg) holds
//                 head c's output channels [D/4 kg, D/4 (kg+1)).
#include <stdlib.h>

#include <type_traits>

#include "pa_device.h"
#include "pa_encode.h"
#include "pa_fp4.h"
#include "pa_launch.h"
#include "pa_tile.h"

namespace pa {

constexpr float kRescale = 8.0f;  // lazy-rescale threshold, log2 units

// LDS of the FP4 kernel, in floats, for GP head columns (shared by the kernel and its
// launch): the q copy ([D + D/DL rows][GP], DL = D / 4).
template <int D, int GP>
constexpr int fp4_qlds_floats() { return (D + 4) * GP; }
// words of one wave's block-id slot (FP4 kernel)
constexpr int kIdsLds = 64;


// Words 1 and 2 of an FP4 outlier record (channels 4 .. 11), wave-uniform. A record no
// wave writes during the launch is read through the scalar cache (no vector-memory wait,
// so a double-buffered tile's loads stay in flight). The record of the tile this wave
// wrote itself in this launch (fresh) is read with a vector load: scalar loads assume
// memory that is constant for the whole dispatch, and a fence does not order them.
__device__ __forceinline__ uint2 record_words12(const uint8_t* rec, bool fresh) {
  if (fresh) {  // the record is 16-byte aligned
    const uint4 r = *reinterpret_cast<const uint4*>(rec);
    return make_uint2((uint32_t)__builtin_amdgcn_readfirstlane((int)r.y),
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)r.z));
  }
  const uint4 r = load_uniform16(rec);
  return make_uint2(r.y, r.z);
}

// pa_append_decode: the workgroup that reads sequence s's last position writes the
// sequence's new row there first, for its kv head, exactly as the cache-write kernels
// store it (16-bit copy, FP8 with the head's scale, FP8 with the row's own scale), by a
// group of 2 R consecutive lanes (aligned to 2 R; t = the lane's place in the group): K on
// places [0, R), V on [R, 2R). `row` indexes the new rows: k_new / v_new hold
// [row][Hkv][D]. Loading (append_load) and storing (append_store) are separate steps, so
// that a wave can have the loads of several rows in flight before it stores any.
template <int KV, int D>
constexpr int append_lanes() { return 2 * (is_f8(KV) ? D / 16 : D * 2 / 16); }
struct NewRow {
  uint4 lo, hi;  // the lane's 16 (FP8 pools: 2 x 8) input values of the row
};
template <int KV, int D>
__device__ __forceinline__ NewRow append_load(const DecodeArgs& a, int row, int kvh, int t) {
  constexpr int R = append_lanes<KV, D>() / 2;  // lanes per row and side
  static_assert(2 * R <= 64, "one wave writes the row");
  const bool vside = t >= R;
  const int c = t - (vside ? R : 0);
  const uint4* src = reinterpret_cast<const uint4*>(vside ? a.v_new : a.k_new) +
                     ((int64_t)row * a.num_kv_heads + kvh) * (D * 2 / 16);
  NewRow r;
  if constexpr (KV == KV_F16 || KV == KV_BF16) {
    r.lo = src[c];
    r.hi = r.lo;
  } else {
    r.lo = src[2 * c];
    r.hi = src[2 * c + 1];
  }
  return r;
}
template <int KV, int D, bool QBF>
__device__ __forceinline__ void append_store(const DecodeArgs& a, const NewRow& r, int kvh,
                                             int b, int off, int t) {
  using G_ = Geo<KV, D>;
  constexpr int R = append_lanes<KV, D>() / 2;
  const bool vside = t >= R;
  const int c = t - (vside ? R : 0);
  const int64_t bh = (int64_t)b * a.num_kv_heads + kvh;
  uint8_t* tile = reinterpret_cast<uint8_t*>(const_cast<void*>(vside ? a.v : a.k)) +
                  bh * (vside ? G_::VTILEB : G_::TILEB);
  if constexpr (KV == KV_F16 || KV == KV_BF16) {
    reinterpret_cast<uint4*>(tile + off * G_::ROWB)[c] = r.lo;
  } else {
    constexpr bool E5 = f8_e5(KV);
    float sc;
    if constexpr (f8_tok(KV)) {
      // the row's absmax over its R threads (consecutive lanes, R divides 64)
      const uint32_t w[8] = {r.lo.x, r.lo.y, r.lo.z, r.lo.w, r.hi.x, r.hi.y, r.hi.z, r.hi.w};
      float mx = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e)
        mx = fmaxf(mx, __builtin_fabsf(act_to_f32<QBF>((w[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu)));
#pragma unroll
      for (int o = R / 2; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      sc = mx / (E5 ? 57344.0f : 448.0f);
      // both token scales live in the K run (K's, then V's)
      if (c == 0)
        reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(const_cast<void*>(a.k)) +
                                 bh * G_::TILEB +
                                 (vside ? PA_FP8T_VSCALE_OFF(D) : PA_FP8T_SCALE_OFF(D)))[off] = sc;
    } else {
      sc = vside ? a.v_scale[kvh] : a.k_scale[kvh];
    }
    const bool fast = __builtin_fabsf(sc) >= 0x1p-80f && __builtin_fabsf(sc) <= 0x1p100f;
    const uint4 codes = fp8_encode16<QBF, E5>(r.lo, r.hi, sc, fast);
    if (vside)
      f8_v_store16<D>(tile, off, c, codes);  // V runs are stored by channel
    else
      *reinterpret_cast<uint4*>(tile + off * D + 16 * c) = codes;
  }
}

// The same for an FP4 pool, by one wave, K then V: a block whose record is still unset gets
// its outlier set from this row alone (the rows a cache-write call of one token per
// sequence puts into a block), then the row is encoded with the block's set; the wave is
// the only writer of the block in this launch, so the V nibbles merge by read-modify-write.
template <int D, bool QBF>
__device__ __forceinline__ void append_row_fp4(const DecodeArgs& a, int s, int kvh, int b,
                                               int off) {
  using TL = Fp4Tile<D>;
  const int lane = threadIdx.x & 63;
  const int64_t bh = (int64_t)b * a.num_kv_heads + kvh;
#pragma unroll
  for (int side = 0; side < 2; ++side) {
    const uint16_t* row = reinterpret_cast<const uint16_t*>(side ? a.v_new : a.k_new) +
                          ((int64_t)s * a.num_kv_heads + kvh) * D;
    uint8_t* tile = reinterpret_cast<uint8_t*>(const_cast<void*>(side ? a.v : a.k)) +
                    bh * TL::kBytes;
    uint16_t* ov = const_cast<uint16_t*>(side ? a.v_out_val : a.k_out_val) +
                   bh * (a.cap - 1) * kBlock;
    const uint4 r4 = *reinterpret_cast<const uint4*>(tile + TL::kRecord);
    uint32_t rw[3] = {r4.x, r4.y, r4.z};
    if ((rw[0] & 0xFFu) == 0xFFu) {  // the block's first write (uniform)
      fp4_calibrate_row<QBF, D>(row, a.cap, rw);
      if (lane == 0) {
        uint32_t* w = reinterpret_cast<uint32_t*>(tile + TL::kRecord);
        w[0] = rw[0];
        w[1] = rw[1];
        w[2] = rw[2];
      }
    }
    int count = (int)(rw[0] & 0xFFu);
    if (count > a.cap) count = a.cap;
    Fp4VBits vb;
    fp4_encode_row<QBF, D>(row, tile, ov, off, side == 1, rw, count, vb);
    if (vb.word) *vb.word = (*vb.word & ~vb.mask) | vb.bits;
  }
}

// The decode of one workgroup. DB selects the block loop: false keeps one tile in flight
// (the next tile is loaded after the current one is consumed; the other waves of the
// compute unit cover the latency), true double-buffers (the next tile's loads are issued
// before the current tile's math, so each wave keeps a tile in flight while it computes).
// PROBE keeps every load of the decode (block ids, tiles, scales, records) and drops the
// arithmetic: each tile's words are XORed into one word per wave, stored to a.sink; the
// time of that launch is what the decode's memory traffic alone costs.
template <int KV, int D, bool QBF, int GP, bool DB, bool APPEND = false, bool PROBE = false>
__device__ __forceinline__ void decode_body(const DecodeArgs& a) {
  using G_ = Geo<KV, D>;
  constexpr int KS = G_::KS, NT = G_::NT, DL = G_::DL;
  // the FP4 q copy holds GP head columns (GP = 8 or 16 >= the GQA group)
  constexpr int kQLds = fp4_qlds_floats<D, GP>();
  static_assert(!DB || KV == KV_FP4, "the double-buffered loop is the FP4 kernel's");
  static_assert(kQLds == (D + D / DL) * GP, "FP4 LDS layout");
  // PV MFMA in bf16 for bf16 pools and where P takes a token scale (p s_t may leave fp16's
  // range), else in fp16: E4M3 and E5M2 codes are fp16 values, and P's hi + lo pair then
  // carries 22 bits at fewer instructions
  constexpr bool PVB = KV == KV_BF16 || tok_scaled(KV);
  // FP4 with G <= 8 (GP = 8): MFMA columns 8..15 repeat heads 0..7 (the same q, hence the
  // same logits, maxima and P); there the B operand of PV is P's low half, so one MFMA per
  // 16 channels carries hi and lo, and the two column halves are added at the end
  constexpr bool SPARE = KV == KV_FP4 && GP == 8 && !PROBE;
  constexpr bool kStreamK = KV != KV_F16 && KV != KV_BF16;  // non-temporal K tile loads
  extern __shared__ float smem[];

  const int lane = threadIdx.x & 63;
  // wave index, pinned as wave-uniform (the compiler cannot prove threadIdx.x / 64 is)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int c = lane & 15;  // MFMA column: query head (QK, PV); K row token; V channel group
  const int kg = lane >> 4;
  // grid.x = kv head fastest, then partition: the workgroups of one
  // block's kv heads run side by side and read neighbouring tiles ([block][kv head][16][D]
  // is contiguous); grid.y = sequence
  const int kvh = (int)(blockIdx.x % (unsigned)a.num_kv_heads);
  const int p = (int)(blockIdx.x / (unsigned)a.num_kv_heads);
  const int s = blockIdx.y;
  const int G = a.group;
  const int Hq = a.num_q_heads;

  const int L = a.context_lens[s];
  const int cap_tokens = a.max_blocks * kBlock;
  const bool split = a.partition_size > 0;
  if (L < 1 || L > cap_tokens || (APPEND && L < a.new_tokens)) {
    if (threadIdx.x == 0 && p == 0 && kvh == 0 && a.err) atomicOr(a.err, PA_DEVERR_BAD_CONTEXT);
    if (PROBE) return;  // the probe has no outputs
    if (!split && p == 0) {
      for (int i = threadIdx.x; i < G * D; i += blockDim.x)
        a.out[((int64_t)s * Hq + kvh * G) * D + i] = 0.0f;
    }
    // split: every partition of the sequence reads as empty (lse -inf, zero output), so a
    // merge over any number of them gives a zero output and lse -inf
    if (split && (int)threadIdx.x < G) {
      const int64_t row = ((int64_t)s * Hq + kvh * G + threadIdx.x) * a.max_partitions + p;
      a.part_lse[row] = -INFINITY;
      for (int i = 0; i < D; ++i) a.part_out[row * D + i] = 0.0f;
    }
    return;
  }
  // the blocks this wave reads: its share of the partition, blocks w, w + W, ...
  const int start = split ? p * a.partition_size : 0;
  if (start >= L) return;  // empty partition: not written, the merge skips it
  const int end = split ? min(start + a.partition_size, L) : L;
  const int jb0 = start / kBlock;

  // APPEND: whether this wave wrote new rows, and the first of its blocks that holds one
  // (it fences before loading that tile); both wave-uniform
  bool wrote = false;
  int first_jb = 0;
  if constexpr (APPEND) {
    // The sequence's new rows go to positions L - n .. L - 1. The wave that will read a
    // position (the partition's blocks go round-robin to the workgroup's waves) writes the
    // new row there first. No other wave or workgroup reads those (block, kv head) tiles in
    // this launch, and they are the last blocks of the sequence, so this wave's last
    // tiles: a fence at workgroup scope just before the first of them is enough (its
    // release waits for the stores to reach L2, its acquire orders the later loads after
    // them), and by then the stores have long completed, so the wait costs nothing. The
    // other waves do not wait. (A device-scope fence would also write back and invalidate
    // the XCD's L2: measured, that cost the FP8 decode of 256 x 8192 tokens 60% of its
    // speed.)
    const int n = a.new_tokens;
    const int lo = max(L - n, start), hi = end;  // this partition's new positions
    if (lo < hi) {
      const int jb_lo = lo / kBlock, jb_hi = (hi - 1) / kBlock;
      first_jb = jb_lo + ((wave - (jb_lo - jb0)) % W + W) % W;
      wrote = first_jb <= jb_hi;
    }
  }
  auto write_new_rows = [&] {
    if constexpr (APPEND) {
      if (!wrote) return;
      const int n = a.new_tokens;
      const int lo = max(L - n, start), hi = end;
      if constexpr (KV == KV_FP4) {
        // (one new row per sequence: position L - 1, the whole wave)
        const int32_t b = a.block_tables[(int64_t)s * a.max_blocks + (L - 1) / kBlock];
        if ((unsigned)b < (unsigned)a.num_blocks)
          append_row_fp4<D, QBF>(a, s, kvh, b, (L - 1) % kBlock);
        else if (lane == 0 && a.err)
          atomicOr(a.err, PA_DEVERR_BAD_BLOCK);
      } else {
        // groups of 2 R lanes, one new row each, every row of this wave's blocks; two rows
        // per group and trip, both loaded before either is stored
        constexpr int LPR = append_lanes<KV, D>(), RPP = 64 / LPR;
        const int g = lane / LPR, t = lane % LPR;
        for (int p0 = lo; p0 < hi; p0 += 2 * RPP) {
          int pos[2];
          bool mine[2];
          int32_t b[2];
          NewRow r[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            pos[k] = p0 + k * RPP + g;
            mine[k] = pos[k] < hi && (pos[k] / kBlock - jb0) % W == wave;
            if (mine[k]) {
              b[k] = a.block_tables[(int64_t)s * a.max_blocks + pos[k] / kBlock];
              r[k] = append_load<KV, D>(a, s * n + (pos[k] - (L - n)), kvh, t);
            }
          }
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            if (mine[k]) {
              if ((unsigned)b[k] < (unsigned)a.num_blocks)
                append_store<KV, D, QBF>(a, r[k], kvh, b[k], pos[k] % kBlock, t);
              else if (t == 0 && a.err)
                atomicOr(a.err, PA_DEVERR_BAD_BLOCK);
            }
          }
        }
      }
    }
  };
  const int nblk = (end + kBlock - 1) / kBlock - jb0;
  const int my_n = wave < nblk ? (nblk - wave + W - 1) / W : 0;

  // ---- block ids ----
  // Single buffer: 64 of this wave's block ids per register, one register ahead, read
  // with readlane. Double buffer: the same 64-id chunks staged in this wave's LDS slot
  // and each id read one block ahead, so that no vector load of ids is pending when the
  // next tile's loads are issued and no scalar load is pending during a block's math (a
  // scalar load may complete out of order, so any wait on LDS would wait for it too).
  // The first chunks are requested before anything else: the first tile's loads wait for
  // them, and the new rows' writes and the query loads go out meanwhile.
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks + jb0 + wave;
  auto load_ids = [&](int chunk) -> int {
    const int x = chunk * 64 + lane;
    return x < my_n ? bt[(int64_t)x * W] : 0;
  };
  int ids_a = load_ids(0), ids_b = load_ids(1), nid_v = 0;

  write_new_rows();

  // ---- query fragments (B operand of S^T = K Q^T), zero for padded heads ----
  uint4 qf[KS];
  if constexpr (PROBE) {  // no query is passed to the probe
#pragma unroll
    for (int t = 0; t < KS; ++t) qf[t] = make_uint4(0, 0, 0, 0);
  } else {
    const int hc = SPARE ? (c & 7) : c;  // the head of MFMA column c
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q) +
                          (((int64_t)s * Hq + kvh * G + hc) * D + DL * kg) * 2;
#pragma unroll
    for (int t = 0; t < KS; ++t)
      qf[t] = hc < G ? reinterpret_cast<const uint4*>(qrow)[t] : make_uint4(0, 0, 0, 0);
  }
  // FP4 only: q in fp32 for the K-outlier term, channel-major: head c of channel ch at
  // (ch + ch / DL) * GP + c. A column's heads are consecutive words (one read per outlier
  // is conflict-free) and the pad of GP words after each DL channels puts the four lane
  // groups of a write on different banks.
  // (staged after the first tile's loads are out: the barrier waits for wave 0's query)
  float* const q_lds = smem;
  auto stage_q = [&] {
    if constexpr (KV == KV_FP4) {
      if (wave == 0) {
#pragma unroll
        for (int t = 0; t < KS; ++t) {
          const uint32_t w[4] = {qf[t].x, qf[t].y, qf[t].z, qf[t].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t b16 = (w[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
            if (c < GP) q_lds[(DL * kg + 8 * t + e + kg) * GP + c] = act_to_f32<QBF>(b16);
          }
        }
      }
      __syncthreads();
    }
  };

  // ---- scale of the logits (base 2) ----
  float cz = a.sm_scale_log2;
  if constexpr (head_scaled(KV)) cz *= a.k_scale[kvh];

  int* const ids_lds = reinterpret_cast<int*>(smem + kQLds) + wave * kIdsLds;
  if constexpr (DB) {
    ids_lds[lane] = ids_a;
    nid_v = ids_lds[0];
  }

  const uint8_t* kpool = reinterpret_cast<const uint8_t*>(a.k);
  const uint8_t* vpool = reinterpret_cast<const uint8_t*>(a.v);
  const int k_lane_off = c * G_::ROWB + kg * G_::KLANEB;
  const int v_lane_off = 4 * kg * G_::ROWB + c * G_::VLANEB;

  // Device-side error bits seen by this wave. They are kept wave-uniform and flagged
  // once at the end: a lane-divergent branch inside the block loop would make the
  // compiler carry the loop's scalar values (block ids, FP4 records) in vector
  // registers, and wait for every scalar load as soon as it is issued.
  int err_bits = 0;
  auto load_tile = [&](Tile<KV, D>& T, int x) {
    if constexpr (APPEND) {
      if (wrote && jb0 + wave + x * W == first_jb) {  // the first tile holding a new row
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      }
    }
    int b_raw;
    if constexpr (DB) {
      b_raw = __builtin_amdgcn_readfirstlane(nid_v);
      if (((x + 1) & 63) == 0) {  // the next chunk replaces this one in the slot
        ids_lds[lane] = ids_b;
        ids_b = load_ids(((x + 1) >> 6) + 1);
      }
      nid_v = ids_lds[(x + 1) & 63];
    } else {
      if (x > 0 && (x & 63) == 0) {
        ids_a = ids_b;
        ids_b = load_ids((x >> 6) + 1);
      }
      b_raw = __builtin_amdgcn_readlane(ids_a, x & 63);
    }
    T.jb = jb0 + wave + x * W;
    T.fresh = APPEND && wrote && T.jb >= first_jb;
    T.ok = (unsigned)b_raw < (unsigned)a.num_blocks;
    err_bits |= T.ok ? 0 : PA_DEVERR_BAD_BLOCK;
    const int b = T.ok ? b_raw : 0;
    T.tile = (int64_t)b * a.num_kv_heads + kvh;
    // each tile is read once per launch: streaming (non-temporal) loads (FP8, 256 x 8192
    // tokens: 94.1 -> 89.7 us). 16-bit K excepted: a lane reads its 64-byte row segment in four 16-byte
    // loads, and with the hint a line can leave before the later loads reach it (the
    // 8B-shaped bf16 workload: 205 -> 274 us); its V loads, each a whole row across 16
    // lanes, stream (209 -> 195 us).
    load_words<G_::KW, kStreamK>(T.k, kpool + T.tile * G_::TILEB + k_lane_off);
    if constexpr (KV == KV_FP4) {
      // one chunk: channels NT c .. NT c + NT - 1 of tokens 4 kg .. 4 kg + 3
      fp4_v_chunk<D, true>(T, vpool + T.tile * G_::TILEB, c, kg);
    } else if constexpr (is_f8(KV)) {
      f8_v_chunk<KV, D, true>(T, vpool + T.tile * G_::VTILEB, c, kg);  // the same chunk
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        load_words<G_::VW, true>(T.v[r], vpool + T.tile * G_::VTILEB + v_lane_off + r * G_::ROWB);
    }
    if constexpr (f8_tok(KV)) {  // per-token scales of tokens 4 kg .. 4 kg + 3
      T.sk = reinterpret_cast<const float4*>(kpool + T.tile * G_::TILEB + PA_FP8T_SCALE_OFF(D))[kg];
      T.sv = reinterpret_cast<const float4*>(kpool + T.tile * G_::TILEB + PA_FP8T_VSCALE_OFF(D))[kg];
    }
    if constexpr (KV == KV_FP4) {
      const uint8_t* kt = kpool + T.tile * G_::TILEB;
      const uint8_t* vt = vpool + T.tile * G_::TILEB;
      T.sk = reinterpret_cast<const float4*>(kt + PA_FP4_SCALE_OFF(D))[kg];
      T.sv = reinterpret_cast<const float4*>(vt + PA_FP4_SCALE_OFF(D))[kg];
      // first word of each outlier record (count and the first three channels): lanes
      // 0-31 read K's, lanes 32-63 V's, into one register; a vector load, so that no
      // scalar load is in flight during the previous tile's math
      T.r0 = *reinterpret_cast<const uint32_t*>((lane < 32 ? kt : vt) + PA_FP4_RECORD_OFF(D));
      // the first outlier slot is part of the tile; its bytes are used only if the
      // record's count is at least 1
      T.k_o0 = reinterpret_cast<const uint2*>(kt + PA_FP4_SLOT0_OFF(D))[kg];
      T.v_o0 = reinterpret_cast<const uint2*>(vt + PA_FP4_SLOT0_OFF(D))[kg];
    }
  };

  // ---- online softmax state ----
  float m = -INFINITY;  // running max (base-2 logits) of head c, same in its 4 lanes
  float l = 0.0f;       // this lane's part of the running sum
  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  bool started = false;  // wave-uniform: a block has been folded into (m, l, acc)

  uint32_t probe_x = 0u;  // PROBE: XOR of every loaded word

  // One block. kFull (a compile-time tag) says the block is in range and all 16 of its
  // tokens are inside the partition, which holds for every block but the last one of a
  // partition; that version carries no per-token masks.
  auto compute = [&](Tile<KV, D>& T, auto kFull) {
    constexpr bool FULL = decltype(kFull)::value;
    if constexpr (PROBE) {
#pragma unroll
      for (int i = 0; i < G_::KW; ++i) probe_x ^= T.k[i];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < G_::VW; ++i) probe_x ^= T.v[r][i];
      if constexpr (tok_scaled(KV))
        probe_x ^= __float_as_uint(T.sk.x + T.sk.y + T.sk.z + T.sk.w + T.sv.x + T.sv.y +
                                   T.sv.z + T.sv.w);
      if constexpr (KV == KV_FP4) probe_x ^= T.r0 ^ T.k_o0.x ^ T.k_o0.y ^ T.v_o0.x ^ T.v_o0.y;
      return;
    }
    const int tok0 = T.jb * kBlock + 4 * kg;
    bool valid[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) valid[r] = FULL || (T.ok && (tok0 + r < end));
    // V bytes of tokens past the context are arbitrary: zeroed, as a NaN code times p = 0
    // would still be NaN (E2M1 has no NaN code)
    if constexpr (!FULL && is_f8(KV)) {  // byte r of every word is token 4 kg + r
      const uint32_t keep = (valid[0] ? 0xFFu : 0u) | (valid[1] ? 0xFF00u : 0u) |
                            (valid[2] ? 0xFF0000u : 0u) | (valid[3] ? 0xFF000000u : 0u);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int i = 0; i < G_::VW; ++i) T.v[r][i] &= keep;
      }
    } else if constexpr (!FULL && KV != KV_FP4) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int i = 0; i < G_::VW; ++i) T.v[r][i] = valid[r] ? T.v[r][i] : 0u;
      }
    }

    // logits S^T[token 4 kg + r][head c]
    f32x4 sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < KS; ++t) sacc = mfma_k32(k_fragment<KV, D, QBF>(T, t), qf[t], sacc, QBF);
    float z[4];
    if constexpr (KV == KV_FP4) {
      const float sk[4] = {T.sk.x, T.sk.y, T.sk.z, T.sk.w};
      float ok[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      // The record sits in scalar registers, so the channel indices below are
      // wave-uniform.
      uint32_t rw[3] = {(uint32_t)__builtin_amdgcn_readlane((int)T.r0, 0), 0u, 0u};
      int nk = (int)(rw[0] & 0xFFu);
      if (nk > 3 && nk != 0xFF) {  // more channels than the first word holds (rare)
        const uint2 r = record_words12(kpool + T.tile * G_::TILEB + PA_FP4_RECORD_OFF(D), T.fresh);
        rw[1] = r.x;
        rw[2] = r.y;
      }
      if (nk == 0xFF) {
        err_bits |= T.ok ? PA_DEVERR_UNCALIBRATED : 0;
        nk = 0;
      }
      if (nk > a.cap) nk = a.cap;
      for (int j = 0; j < nk; ++j) {
        const int pos = 1 + j;
        const int ch = (int)((rw[pos >> 2] >> ((pos & 3) * 8)) & 0xFFu);
        // padding heads read some real column: their logits are never used
        const float qv = q_lds[(ch + ch / DL) * GP + (c & (GP - 1))];
        const uint2 ov = j == 0 ? T.k_o0
                                : *reinterpret_cast<const uint2*>(
                                      a.k_out_val + ((T.tile * (a.cap - 1) + (j - 1)) * kBlock +
                                                     4 * kg));
        ok[0] = __builtin_fmaf(qv, f16_bits_to_f32(ov.x & 0xFFFFu), ok[0]);
        ok[1] = __builtin_fmaf(qv, f16_bits_to_f32(ov.x >> 16), ok[1]);
        ok[2] = __builtin_fmaf(qv, f16_bits_to_f32(ov.y & 0xFFFFu), ok[2]);
        ok[3] = __builtin_fmaf(qv, f16_bits_to_f32(ov.y >> 16), ok[3]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
        z[r] = valid[r] ? __builtin_fmaf(sacc[r], sk[r], ok[r]) * cz : -INFINITY;
    } else if constexpr (f8_tok(KV)) {
      const float sk[4] = {T.sk.x, T.sk.y, T.sk.z, T.sk.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) z[r] = valid[r] ? sacc[r] * sk[r] * cz : -INFINITY;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) z[r] = valid[r] ? sacc[r] * cz : -INFINITY;
    }

    // online softmax (base 2), lazy rescale
    const float mb = group4_max(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
    if (__builtin_amdgcn_ballot_w64(mb > m + kRescale) != 0) {  // wave-uniform
      const float mn = fmaxf(m, mb);
      if (started) {  // before the first block l and acc are all zero
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        l *= alpha;
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[n] *= alpha;
      }
      m = mn;
    }
    started = true;
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[r] = valid[r] ? __builtin_amdgcn_exp2f(z[r] - m) : 0.0f;
      l += pr[r];
    }

    // P^T operand: hi + lo 16-bit pairs (per-token formats: p * s_t, the V token scale)
    float pv[4];
    if constexpr (tok_scaled(KV)) {
      const float sv[4] = {T.sv.x, T.sv.y, T.sv.z, T.sv.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) pv[r] = valid[r] ? pr[r] * sv[r] : 0.0f;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) pv[r] = pr[r];
    }
    uint32_t h01, h23, l01, l23;
    split2(pv[0], pv[1], PVB, h01, l01);
    split2(pv[2], pv[3], PVB, h23, l23);
    const uint2 ph = make_uint2(h01, h23), pl = make_uint2(l01, l23);

    if constexpr (KV == KV_FP4) {
      // V outliers: out[c][ch] += sum_t p_t * o_t,ch (fp16 values, unscaled p); ch is
      // wave-uniform (the record sits in scalar registers). Each term goes straight into
      // its accumulator register, before this block's PV MFMAs, so the indexed register
      // read waits only for the previous block's.
      uint32_t rw[3] = {(uint32_t)__builtin_amdgcn_readlane((int)T.r0, 32), 0u, 0u};
      int nv = (int)(rw[0] & 0xFFu);
      if (nv > 3 && nv != 0xFF) {
        const uint2 r = record_words12(vpool + T.tile * G_::TILEB + PA_FP4_RECORD_OFF(D), T.fresh);
        rw[1] = r.x;
        rw[2] = r.y;
      }
      if (nv == 0xFF) {
        err_bits |= T.ok ? PA_DEVERR_UNCALIBRATED : 0;
        nv = 0;
      }
      if (nv > a.cap) nv = a.cap;
      for (int j = 0; j < nv; ++j) {
        const int pos = 1 + j;
        const int ch = (int)((rw[pos >> 2] >> ((pos & 3) * 8)) & 0xFFu);
        const uint2 ov = j == 0 ? T.v_o0
                                : *reinterpret_cast<const uint2*>(
                                      a.v_out_val + ((T.tile * (a.cap - 1) + (j - 1)) * kBlock +
                                                     4 * kg));
        // slots of tokens past the context hold arbitrary bits (maybe NaN): masked
        const float o4[4] = {valid[0] ? f16_bits_to_f32(ov.x & 0xFFFFu) : 0.0f,
                             valid[1] ? f16_bits_to_f32(ov.x >> 16) : 0.0f,
                             valid[2] ? f16_bits_to_f32(ov.y & 0xFFFFu) : 0.0f,
                             valid[3] ? f16_bits_to_f32(ov.y >> 16) : 0.0f};
        float part = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) part = __builtin_fmaf(pr[r], o4[r], part);
        part = group4_sum(part);
        // channel ch is entry ch % DL = NT r + n, in acc[n][r], of the lanes with
        // kg = ch / DL
        // (SPARE: the low-half columns 8..15 take no outlier term)
        add_entry<NT>(acc, ch % DL, kg == ch / DL && (!SPARE || c < 8) ? part : 0.0f);
      }
    }
    uint2 vf[NT];
    v_fragments<KV, D, PVB>(T, vf);
    if constexpr (SPARE) {
      const uint2 pb = c < 8 ? ph : pl;
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n] = mfma_k16(vf[n], pb, acc[n], PVB);
    } else {
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        acc[n] = mfma_k16(vf[n], ph, acc[n], PVB);
        acc[n] = mfma_k16(vf[n], pl, acc[n], PVB);
      }
    }
  };

  // ---- block loop (single or double buffered, see DB) ----
  // Every block of the loop body is full: a partition starts on a block boundary, so only
  // its last block can end early, and that block is the last one of some wave's run. It
  // is handled after the loop with per-token masks. A block whose id is out of range is
  // skipped (and flagged).
  if constexpr (DB) {
    Tile<KV, D> ta, tb;
    if (my_n > 0) load_tile(ta, 0);
    stage_q();
    int i = 0;
    for (; i + 2 < my_n; i += 2) {
      load_tile(tb, i + 1);
      if (ta.ok) compute(ta, std::true_type{});
      load_tile(ta, i + 2);
      if (tb.ok) compute(tb, std::true_type{});
    }
    if (i + 2 == my_n) {
      load_tile(tb, i + 1);
      if (ta.ok) compute(ta, std::true_type{});
      if (tb.ok) compute(tb, std::false_type{});
    } else if (my_n > 0 && ta.ok) {
      compute(ta, std::false_type{});
    }
  } else {
    Tile<KV, D> tile;
    if (my_n > 0) load_tile(tile, 0);
    stage_q();
    for (int i = 0; i + 1 < my_n; ++i) {
      if (tile.ok) compute(tile, std::true_type{});
      load_tile(tile, i + 1);
    }
    if (my_n > 0 && tile.ok) compute(tile, std::false_type{});
  }

  // ---- epilogue ----
  if (err_bits != 0 && lane == 0 && a.err) atomicOr(a.err, err_bits);
  if constexpr (PROBE) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) probe_x ^= (uint32_t)__shfl_xor((int)probe_x, o);
    if (lane == 0 && probe_x != 0u)
      atomicXor(a.sink + ((blockIdx.y * gridDim.x + blockIdx.x) * 8u + (unsigned)wave) % 1024u,
                probe_x);
    return;
  }
  if constexpr (SPARE) {
    // column c < 8 adds column c + 8 (the same head's P-low products): rotate each 16-lane
    // row by 8
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc[n][r] += __int_as_float(__builtin_amdgcn_update_dpp(
            0, __float_as_int(acc[n][r]), 0x128 /* row_ror:8 */, 0xF, 0xF, false));
  }
  const float lt = group4_sum(l);
  const float vscale = head_scaled(KV) ? a.v_scale[kvh] : 1.0f;
  const int h = kvh * G + c;
  if (W == 1) {
    if (c < G) {
      const float inv = lt > 0.0f ? vscale / lt : 0.0f;  // 0: every block id was bad
      float* dst = split ? a.part_out + (((int64_t)s * Hq + h) * a.max_partitions + p) * D
                         : a.out + ((int64_t)s * Hq + h) * D;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int n = 0; n < NT; ++n) dst[DL * kg + NT * r + n] = acc[n][r] * inv;
      if (split && kg == 0)
        a.part_lse[((int64_t)s * Hq + h) * a.max_partitions + p] = (m + __log2f(lt)) * kLn2;
    }
    return;
  }

  // W > 1: merge the waves' states in LDS. FP4: the merge reuses the LDS of the q copy and
  // the id slots, so every wave must be past its block loop first (the merge then costs no
  // LDS of its own, and a 2-wave workgroup keeps the occupancy of two 1-wave ones).
  constexpr int STRIDE = DL + 4;  // floats per lane record (padded)
  if constexpr (KV == KV_FP4) __syncthreads();
  float* m_lds = smem;
  float* l_lds = m_lds + 16 * 8;
  float* acc_lds = l_lds + 16 * 8;  // [W][64][STRIDE]
  if (kg == 0) {
    m_lds[wave * 16 + c] = m;
    l_lds[wave * 16 + c] = lt;
  }
  float* mine = acc_lds + ((int64_t)wave * 64 + lane) * STRIDE;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int n = 0; n < NT; ++n) mine[NT * r + n] = acc[n][r];
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * (D / 4); idx += blockDim.x) {
    const int g = idx / (D / 4);
    const int d = (idx % (D / 4)) * 4;
    float M = -INFINITY;
    for (int w = 0; w < W; ++w) M = fmaxf(M, m_lds[w * 16 + g]);
    float Lsum = 0.0f;
    float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    const int src_lane = g + 16 * (d / DL);
    const int e = d % DL;
    for (int w = 0; w < W; ++w) {
      // 0 for a wave with nothing folded in (idle, or every block id bad): m = -inf, and
      // -inf - -inf would be NaN when no wave has anything
      const float mw = m_lds[w * 16 + g];
      const float f = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
      Lsum += f * l_lds[w * 16 + g];
      const float4 x = *reinterpret_cast<const float4*>(acc_lds + ((int64_t)w * 64 + src_lane) * STRIDE + e);
      o.x += f * x.x;
      o.y += f * x.y;
      o.z += f * x.z;
      o.w += f * x.w;
    }
    const float inv = Lsum > 0.0f ? vscale / Lsum : 0.0f;
    o.x *= inv;
    o.y *= inv;
    o.z *= inv;
    o.w *= inv;
    const int hh = kvh * G + g;
    float* dst = split ? a.part_out + (((int64_t)s * Hq + hh) * a.max_partitions + p) * D
                       : a.out + ((int64_t)s * Hq + hh) * D;
    *reinterpret_cast<float4*>(dst + d) = o;
    if (split && d == 0)
      a.part_lse[((int64_t)s * Hq + hh) * a.max_partitions + p] = (M + __log2f(Lsum)) * kLn2;
  }
}

// 16-bit and FP8 pools: one tile in flight per wave, occupancy left to the register count
// (5 waves per SIMD for FP8 at head_dim 128).
template <int KV, int D, bool QBF, int GP, bool APPEND = false, bool PROBE = false>
__global__ __launch_bounds__(512) void k_decode(DecodeArgs a) {
  decode_body<KV, D, QBF, GP, false, APPEND, PROBE>(a);
}

// FP4 pools: a tile is half the bytes of an FP8 one, so one tile per wave leaves too little
// in flight; the double-buffered loop, held to at least 4 waves per SIMD (128 registers),
// keeps about twice as much.
template <int D, bool QBF, int GP, bool APPEND = false, bool PROBE = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void k_decode_fp4(
    DecodeArgs a) {
  decode_body<KV_FP4, D, QBF, GP, true, APPEND, PROBE>(a);
}

template <int KV, int D, int GP>
static size_t decode_lds_bytes(int waves) {
  size_t f = KV == KV_FP4 ? fp4_qlds_floats<D, GP>() +
                                (size_t)waves * kIdsLds
                          : 0;
  // the wave merge (FP4: in the same bytes, after the block loops)
  const size_t merge = waves > 1 ? 2 * 16 * 8 + (size_t)waves * 64 * (D / 4 + 4) : 0;
  f = KV == KV_FP4 ? (f > merge ? f : merge) : f + merge;
  return f * sizeof(float);
}

template <int KV, int D, bool QBF, int GP = 16>
static int launch_one(const DecodeArgs& a, int waves, hipStream_t st, bool probe = false) {
  const int P = a.partition_size > 0 ? a.max_partitions : 1;
  // fewer waves per workgroup if their LDS would not fit the device's limit
  int dev = 0, max_lds = 65536;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
          hipSuccess)
    max_lds = 65536;
  while (waves > 1 && decode_lds_bytes<KV, D, GP>(waves) > (size_t)max_lds) waves /= 2;
  const size_t lds = decode_lds_bytes<KV, D, GP>(waves);
  const dim3 grid((unsigned)((int64_t)P * a.num_kv_heads), (unsigned)a.num_seqs, 1);
  if (probe) {
    if constexpr (KV == KV_FP4)
      hipLaunchKernelGGL((k_decode_fp4<D, QBF, GP, false, true>), grid, dim3(64 * waves), lds,
                         st, a);
    else
      hipLaunchKernelGGL((k_decode<KV, D, QBF, GP, false, true>), grid, dim3(64 * waves), lds,
                         st, a);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
  }
  if constexpr (KV == KV_FP4) {
    if (a.k_new)
      hipLaunchKernelGGL((k_decode_fp4<D, QBF, GP, true>), grid, dim3(64 * waves), lds, st, a);
    else
      hipLaunchKernelGGL((k_decode_fp4<D, QBF, GP, false>), grid, dim3(64 * waves), lds, st, a);
  } else if (a.k_new) {
    hipLaunchKernelGGL((k_decode<KV, D, QBF, GP, true>), grid, dim3(64 * waves), lds, st, a);
  } else {
    hipLaunchKernelGGL((k_decode<KV, D, QBF, GP, false>), grid, dim3(64 * waves), lds, st, a);
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int launch_decode(const DecodeArgs& a, int kv, bool qbf, int D, int waves, hipStream_t st) {
  if (D == 128) {
    switch (kv) {
      case KV_F16: return launch_one<KV_F16, 128, false>(a, waves, st);
      case KV_BF16: return launch_one<KV_BF16, 128, true>(a, waves, st);
      case KV_FP8:
        return qbf ? launch_one<KV_FP8, 128, true>(a, waves, st)
                   : launch_one<KV_FP8, 128, false>(a, waves, st);
      case KV_BF8:
        return qbf ? launch_one<KV_BF8, 128, true>(a, waves, st)
                   : launch_one<KV_BF8, 128, false>(a, waves, st);
      case KV_FP8T:
        return qbf ? launch_one<KV_FP8T, 128, true>(a, waves, st)
                   : launch_one<KV_FP8T, 128, false>(a, waves, st);
      case KV_BF8T:
        return qbf ? launch_one<KV_BF8T, 128, true>(a, waves, st)
                   : launch_one<KV_BF8T, 128, false>(a, waves, st);
      case KV_FP4:
        if (a.group <= 8)
          return qbf ? launch_one<KV_FP4, 128, true, 8>(a, waves, st)
                     : launch_one<KV_FP4, 128, false, 8>(a, waves, st);
        return qbf ? launch_one<KV_FP4, 128, true, 16>(a, waves, st)
                   : launch_one<KV_FP4, 128, false, 16>(a, waves, st);
    }
  } else {
    switch (kv) {
      case KV_F16: return launch_one<KV_F16, 64, false>(a, waves, st);
      case KV_BF16: return launch_one<KV_BF16, 64, true>(a, waves, st);
      case KV_FP8:
        return qbf ? launch_one<KV_FP8, 64, true>(a, waves, st)
                   : launch_one<KV_FP8, 64, false>(a, waves, st);
      case KV_BF8:
        return qbf ? launch_one<KV_BF8, 64, true>(a, waves, st)
                   : launch_one<KV_BF8, 64, false>(a, waves, st);
      case KV_FP8T:
        return qbf ? launch_one<KV_FP8T, 64, true>(a, waves, st)
                   : launch_one<KV_FP8T, 64, false>(a, waves, st);
      case KV_BF8T:
        return qbf ? launch_one<KV_BF8T, 64, true>(a, waves, st)
                   : launch_one<KV_BF8T, 64, false>(a, waves, st);
      case KV_FP4:
        if (a.group <= 8)
          return qbf ? launch_one<KV_FP4, 64, true, 8>(a, waves, st)
                     : launch_one<KV_FP4, 64, false, 8>(a, waves, st);
        return qbf ? launch_one<KV_FP4, 64, true, 16>(a, waves, st)
                   : launch_one<KV_FP4, 64, false, 16>(a, waves, st);
    }
  }
  return PA_ERR_DTYPE;
}

// The decode's launch with the arithmetic compiled out (decode_body's PROBE): same grid,
// waves, partitions, block order and loads. The query dtype does not matter there.
int launch_gather_probe(const DecodeArgs& a, int kv, int D, int waves, uint32_t* sink,
                        hipStream_t st) {
  DecodeArgs b = a;
  b.sink = sink;
  b.k_new = b.v_new = nullptr;
  if (D == 128) {
    switch (kv) {
      case KV_F16: return launch_one<KV_F16, 128, false>(b, waves, st, true);
      case KV_BF16: return launch_one<KV_BF16, 128, true>(b, waves, st, true);
      case KV_FP8: return launch_one<KV_FP8, 128, true>(b, waves, st, true);
      case KV_BF8: return launch_one<KV_BF8, 128, true>(b, waves, st, true);
      case KV_FP8T: return launch_one<KV_FP8T, 128, true>(b, waves, st, true);
      case KV_BF8T: return launch_one<KV_BF8T, 128, true>(b, waves, st, true);
      case KV_FP4: return launch_one<KV_FP4, 128, true, 8>(b, waves, st, true);
    }
  } else {
    switch (kv) {
      case KV_F16: return launch_one<KV_F16, 64, false>(b, waves, st, true);
      case KV_BF16: return launch_one<KV_BF16, 64, true>(b, waves, st, true);
      case KV_FP8: return launch_one<KV_FP8, 64, true>(b, waves, st, true);
      case KV_BF8: return launch_one<KV_BF8, 64, true>(b, waves, st, true);
      case KV_FP8T: return launch_one<KV_FP8T, 64, true>(b, waves, st, true);
      case KV_BF8T: return launch_one<KV_BF8T, 64, true>(b, waves, st, true);
      case KV_FP4: return launch_one<KV_FP4, 64, true, 8>(b, waves, st, true);
    }
  }
  return PA_ERR_DTYPE;
}

}  // namespace pa
