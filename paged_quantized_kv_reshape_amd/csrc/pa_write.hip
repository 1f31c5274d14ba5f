// pa_write.hip - cache write ("reshape and cache") kernels for gfx950.
//
// Each new token row goes to its slot = physical_block * 16 + offset of a paged pool
// (xonoai.com field report on vLLM v0.7.2, "Deconstructing the v0.7.2 Architecture";
// inferensys glossary "vLLM", PagedAttention entry), stored as a 16-bit copy, as FP8
// E4M3 codes with a per-head fp32 scale, or as 4-bit E2M1 codes with a per-token scale
// and the block's outlier channels kept in fp16 (dailyaiworld.com, "vLLM 0.7 Ships
// Unified KV Cache Compression", "Technical Breakdown: Dynamic Quantization with Outlier
// Retention", steps 1-3).
//
// Pool tile of (block, kv head): K in 16 token rows, row-major, so one token's row is one
// contiguous run of head_dim values (head_dim / 2 bytes for FP4); 16-bit V likewise, FP8
// and FP4 V codes by channel (a channel's codes for consecutive tokens together, the order
// the P.V product takes them).
#include "pa_device.h"
#include "pa_encode.h"
#include "pa_fp4.h"
#include "pa_launch.h"
#include "pa_tile.h"

namespace pa {

__device__ __forceinline__ void flag(int32_t* err, int32_t bit) {
  if (err) atomicOr(err, bit);
}

// ---------------------------------------------------------------------------------
// 16-bit copy and FP8: one thread per 16-byte input chunk (copy) or per 16 values (FP8)
// of a (token, head) row - of four rows for FP8; consecutive threads walk chunk, then head,
// then token, so a workgroup reads whole token rows. CH = threads per (token, head) row, a
// power of two. The launcher keeps the thread count below 2^31, so the index math is
// 32-bit.
// ---------------------------------------------------------------------------------
template <int CH>
__device__ __forceinline__ bool row_chunk(int32_t T, int32_t hkv, const int64_t* __restrict__ slots,
                                          int64_t nslots, int32_t* err, int64_t& src,
                                          int64_t& dst, int& h) {
  const uint32_t idx = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t per_tok = (uint32_t)hkv * CH;
  const uint32_t i = idx / per_tok;
  const uint32_t rem = idx - i * per_tok;
  const int c = (int)(rem & (CH - 1));
  h = (int)(rem / CH);
  if (i >= (uint32_t)T) return false;
  const int64_t slot = slots[i];
  if (slot < 0) return false;
  if (slot >= nslots) {
    if (c == 0) flag(err, PA_DEVERR_BAD_SLOT);
    return false;
  }
  src = ((int64_t)i * hkv + h) * CH + c;
  dst = (((slot >> 4) * hkv + h) * kBlock + (slot & 15)) * CH + c;
  return true;
}

template <int CH>
__global__ __launch_bounds__(256) void k_write_copy(const uint4* __restrict__ k_new,
                                                    const uint4* __restrict__ v_new,
                                                    uint4* __restrict__ k_pool,
                                                    uint4* __restrict__ v_pool,
                                                    const int64_t* __restrict__ slots,
                                                    int32_t T, int32_t hkv, int64_t nslots,
                                                    int32_t* err) {
  int64_t src, dst;
  int h;
  if (!row_chunk<CH>(T, hkv, slots, nslots, err, src, dst, h)) return;
  k_pool[dst] = k_new[src];
  v_pool[dst] = v_new[src];
}

// FP8 (head or token scales). A V run is stored by channel (a channel's codes for four
// tokens share a word, see f8_v_chunk), so the rows of a call that land in four aligned
// slots 4 q .. 4 q + 3 of one block in order - a prefill chunk's rows do - are written
// together: whole 16-byte V slots (four channels of the four tokens) and their four K rows.
// Any other row is written alone, its V codes byte by byte.
//   One thread per 16 values (chunk c of CH) of a head over a window of four rows
// 4 f .. 4 f + 3; consecutive threads walk chunk, then head, then window. The thread writes
// the four that starts in its window, if any (it may reach three rows past the window),
// and every other row of the window that no four covers. At most one four starts within
// any four rows, so each row is written once.
//   Token scales (TOK): a row's scale is fp32(max |x| / M) (M = 448 or 57344), reduced over
// its CH threads (consecutive lanes of one wave: CH divides 64, every (head, window) starts
// on a multiple of CH, and a group's lanes branch alike); both scales go to the K run.
template <bool BF16, int CH, bool E5, bool TOK>
__global__ __launch_bounds__(256) void k_write_fp8(const uint4* __restrict__ k_new,
                                                   const uint4* __restrict__ v_new,
                                                   uint8_t* __restrict__ k_pool,
                                                   uint8_t* __restrict__ v_pool,
                                                   const float* __restrict__ k_scale,
                                                   const float* __restrict__ v_scale,
                                                   const int64_t* __restrict__ slots,
                                                   int32_t T, int32_t hkv, int64_t nslots,
                                                   int32_t* err) {
  constexpr int D = CH * 16, NT = D / 16;
  constexpr int64_t TB = TOK ? PA_FP8T_TILE_BYTES(D) : 16 * D;
  constexpr int64_t VTB = TOK ? PA_FP8T_VTILE_BYTES(D) : 16 * D;
  constexpr float FMAX = E5 ? 57344.0f : 448.0f;
  const uint32_t idx = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t per_win = (uint32_t)hkv * CH;
  const uint32_t f = idx / per_win;
  const uint32_t rem = idx - f * per_win;
  const int c = (int)(rem & (CH - 1));
  const int h = (int)(rem / CH);
  const int64_t i0 = 4 * (int64_t)f;
  if (i0 >= T) return;  // (a whole (head, window)'s lanes leave together)
  // slots of rows i0 - 3 .. i0 + 6 (-1 outside the call)
  int64_t sl[10];
#pragma unroll
  for (int k = 0; k < 10; ++k) {
    const int64_t i = i0 - 3 + k;
    sl[k] = i >= 0 && i < T ? slots[i] : -1;
  }
  auto four_at = [&](int k) {  // rows i0 - 3 + k .. + 3 fill an aligned four in order
    return sl[k] >= 0 && (sl[k] & 3) == 0 && sl[k] + 3 < nslots && sl[k + 1] == sl[k] + 1 &&
           sl[k + 2] == sl[k] + 2 && sl[k + 3] == sl[k] + 3;
  };
  int lo = 3;  // window rows before lo are covered by a four that starts before the window
#pragma unroll
  for (int k = 0; k < 3; ++k)
    if (four_at(k)) lo = k + 4;
  int mine = 7;  // the four that starts in the window, 7 for none
#pragma unroll
  for (int k = 6; k >= 3; --k)
    if (k >= lo && four_at(k)) mine = k;

  auto scale_of = [&](const uint4 a, const uint4 b, const float* hs) {
    if constexpr (TOK) {
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      float m = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e)
        m = fmaxf(m, __builtin_fabsf(act_to_f32<BF16>((w[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu)));
#pragma unroll
      for (int o = CH / 2; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
      return m / FMAX;
    } else {
      return hs[h];
    }
  };
  auto finite = [](float x) {
    return __builtin_fabsf(x) >= 0x1p-80f && __builtin_fabsf(x) <= 0x1p100f;
  };

  // rows of the window that no four covers, one by one
  for (int k = lo; k < mine && k < 7; ++k) {
    const int64_t slot = sl[k];
    if (slot < 0) continue;  // (also past the end of the call)
    if (slot >= nslots) {
      if (c == 0) flag(err, PA_DEVERR_BAD_SLOT);
      continue;
    }
    const int64_t src = ((i0 - 3 + k) * hkv + h) * CH + c;
    const uint4 k0 = k_new[2 * src], k1 = k_new[2 * src + 1];
    const uint4 v0 = v_new[2 * src], v1 = v_new[2 * src + 1];
    const float sk = scale_of(k0, k1, k_scale), sv = scale_of(v0, v1, v_scale);
    const int64_t bh = (slot >> 4) * hkv + h;
    const int off = (int)(slot & 15);
    uint8_t* const krun = k_pool + bh * TB;
    *reinterpret_cast<uint4*>(krun + off * D + 16 * c) =
        fp8_encode16<BF16, E5>(k0, k1, sk, finite(sk));
    f8_v_store16<D>(v_pool + bh * VTB, off, c, fp8_encode16<BF16, E5>(v0, v1, sv, finite(sv)));
    if (TOK && c == 0) {
      reinterpret_cast<float*>(krun + PA_FP8T_SCALE_OFF(D))[off] = sk;
      reinterpret_cast<float*>(krun + PA_FP8T_VSCALE_OFF(D))[off] = sv;
    }
  }
  if (mine == 7) return;

  // the four rows i0 - 3 + mine .. + 3 into slots s .. s + 3 of one block
  const int64_t s = sl[mine];
  const int64_t bh = (s >> 4) * hkv + h;
  const int off0 = (int)(s & 15);
  uint8_t* const krun = k_pool + bh * TB;
  uint8_t* const vrun = v_pool + bh * VTB;
  uint32_t w[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t src = ((i0 - 3 + mine + r) * hkv + h) * CH + c;
    const uint4 k0 = k_new[2 * src], k1 = k_new[2 * src + 1];
    const uint4 v0 = v_new[2 * src], v1 = v_new[2 * src + 1];
    const float sk = scale_of(k0, k1, k_scale), sv = scale_of(v0, v1, v_scale);
    *reinterpret_cast<uint4*>(krun + (off0 + r) * D + 16 * c) =
        fp8_encode16<BF16, E5>(k0, k1, sk, finite(sk));
    const uint4 vc = fp8_encode16<BF16, E5>(v0, v1, sv, finite(sv));
    w[r][0] = vc.x;
    w[r][1] = vc.y;
    w[r][2] = vc.z;
    w[r][3] = vc.w;
    if (TOK && c == 0) {
      reinterpret_cast<float*>(krun + PA_FP8T_SCALE_OFF(D))[off0 + r] = sk;
      reinterpret_cast<float*>(krun + PA_FP8T_VSCALE_OFF(D))[off0 + r] = sv;
    }
  }
  // V slot i of the chunk: channels 16 c + 4 i .. + 3 of the four tokens, a channel's four
  // token bytes to a word - a 4 x 4 byte transpose of word i of the four rows' codes
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x0 = w[0][i], x1 = w[1][i], x2 = w[2][i], x3 = w[3][i];
    const uint32_t u0 = __builtin_amdgcn_perm(x1, x0, 0x05010400u);  // x0b0 x1b0 x0b1 x1b1
    const uint32_t u1 = __builtin_amdgcn_perm(x1, x0, 0x07030602u);  // x0b2 x1b2 x0b3 x1b3
    const uint32_t y0 = __builtin_amdgcn_perm(x3, x2, 0x05010400u);
    const uint32_t y1 = __builtin_amdgcn_perm(x3, x2, 0x07030602u);
    const uint4 slot16 = make_uint4(__builtin_amdgcn_perm(y0, u0, 0x05040100u),
                                    __builtin_amdgcn_perm(y0, u0, 0x07060302u),
                                    __builtin_amdgcn_perm(y1, u1, 0x05040100u),
                                    __builtin_amdgcn_perm(y1, u1, 0x07060302u));
    const int ch = 16 * c + 4 * i, g = ch / NT, jj = ch % NT;
    *reinterpret_cast<uint4*>(vrun + (jj / 4) * 1024 + (16 * (off0 / 4) + g) * 16) = slot16;
  }
}

// ---------------------------------------------------------------------------------
// FP4 E2M1 + fp16 outliers, three launches per call.
//
// A block's record (16 bytes per block, kv head, K|V) reads 0xFF.. until the block is
// first written. A call calibrates every block it opens on the rows it puts there, so the
// kernels must find, for each such block, the set of this call's rows in it, without
// scratch memory of their own:
//   mark      each row landing in an unset record clears bit `offset` of the record's last
//             word (bytes 12..15, never an index since at most 11 channels are stored)
//             and parks its row index in the tile's scale word for that offset, a word the
//             encode launch overwrites with the row's real scale;
//   calibrate the row with the lowest cleared offset (the leader) reads the row list from
//             the parked indices, computes the outlier set and writes record bytes 0..11;
//             the others only read bytes 12..15, which this launch never writes;
//   encode    every row reads the record (bytes 0..11), stores codes, scale and outliers,
//             and sets bytes 12..15 back to 0xFF.
// grid.z selects K (0) or V (1).
// ---------------------------------------------------------------------------------
struct Fp4Side {
  const uint16_t* rows;  // new rows [T, Hkv, D] (activation bits)
  uint8_t* tiles;        // [NB, Hkv, PA_FP4_TILE_BYTES(D)]: codes, scales, record, slot 0
  uint16_t* out_val;     // [NB, Hkv, CAP - 1, 16]: outlier slots 1 .. CAP - 1
};

struct Fp4Args {
  Fp4Side side[2];
  const int64_t* slots;
  int32_t num_tokens, hkv, head_dim, cap;
  int64_t nslots;
  int32_t* err;
  // per-sequence calibration (k_fp4_adopt): row i belongs to sequence token_seq[i], whose
  // record for (K|V, head h) is seq_records[((seq * 2 + side) * hkv + h) * 16 ...]
  const int32_t* token_seq;
  const uint8_t* seq_records;
  int32_t num_seqs;
};
struct SeqOutlierArgs {
  const uint16_t* k_rows;  // [num_rows, hkv, D] activation bits
  const uint16_t* v_rows;
  const int32_t* row_start;  // [S + 1]
  int64_t num_rows;
  int32_t hkv, cap;
  uint8_t* records;  // [S, 2, hkv, 16]
  int32_t* err;
};

template <int D>
__global__ __launch_bounds__(256) void k_fp4_mark(Fp4Args a) {
  using TL = Fp4Tile<D>;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = (int64_t)a.num_tokens * a.hkv;
  if (idx >= n) return;
  const Fp4Side& sd = a.side[blockIdx.z];
  const int64_t i = idx / a.hkv, h = idx - i * a.hkv;
  const int64_t slot = a.slots[i];
  if (slot < 0) return;
  if (slot >= a.nslots) {
    if (h == 0 && blockIdx.z == 0) flag(a.err, PA_DEVERR_BAD_SLOT);
    return;
  }
  const int64_t bh = (slot >> 4) * a.hkv + h;
  const int off = (int)(slot & 15);
  uint8_t* tile = sd.tiles + bh * TL::kBytes;
  uint8_t* rec = tile + TL::kRecord;
  if (rec[0] != 0xFF) return;  // already calibrated: reuse its channel set
  atomicAnd(reinterpret_cast<unsigned int*>(rec + 12), ~(1u << off));
  reinterpret_cast<int32_t*>(tile + TL::kScale)[off] = (int32_t)i;
}

// One wave per (row, head, K|V); only block leaders do work.
constexpr int kRowsPerWg = 4;  // FP4 calibrate / encode: one wave per row, 4 rows per workgroup
static_assert(kRowsPerWg == 4, "the FP4 encode merges the V codes of a four of tokens");

template <bool BF16, int D>
__global__ __launch_bounds__(64 * kRowsPerWg) void k_fp4_calibrate(Fp4Args a) {
  using TL = Fp4Tile<D>;
  const int i = blockIdx.x * kRowsPerWg + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = blockIdx.y;
  const Fp4Side& sd = a.side[blockIdx.z];
  const int lane = threadIdx.x & 63;
  if (i >= a.num_tokens) return;
  const int64_t slot = a.slots[i];
  if (slot < 0 || slot >= a.nslots) return;
  const int64_t bh = (slot >> 4) * a.hkv + h;
  const int off = (int)(slot & 15);
  uint8_t* tile = sd.tiles + bh * TL::kBytes;
  uint8_t* rec = tile + TL::kRecord;
  const uint32_t pending = ~*reinterpret_cast<const volatile uint32_t*>(rec + 12) & 0xFFFFu;
  if (!(pending & (1u << off))) return;              // not opened by this call
  if (off != __builtin_ctz(pending)) return;          // not the leader
  const int32_t* parked = reinterpret_cast<const int32_t*>(tile + TL::kScale);

  // Per-channel RMS over this call's rows in the block, rows taken in ascending offset.
  // Lane o < 16 fetches the parked row index of offset o and checks it against the slot
  // mapping (a parked index is trusted only if that row really targets this slot: a
  // record that did not start as all 0xFF could carry stray cleared bits); then every
  // row's values are loaded before any is summed, so the loads overlap.
  constexpr int CPL = D / 64;  // channels per lane: lane + 64 * k
  const int64_t blk_base = (slot >> 4) << 4;
  int my_row = -1;
  if (lane < 16 && ((pending >> lane) & 1u)) {
    const int32_t row = parked[lane];
    if (row >= 0 && row < a.num_tokens && a.slots[row] == blk_base + lane) my_row = row;
  }
  const uint32_t rows = (uint32_t)__builtin_amdgcn_ballot_w64(my_row >= 0) & 0xFFFFu;
  if (rows == 0) return;
  const int n = __builtin_popcount(rows);
  float xv[kBlock][CPL];
#pragma unroll
  for (int o = 0; o < kBlock; ++o) {
#pragma unroll
    for (int k = 0; k < CPL; ++k) xv[o][k] = 0.0f;
    if (rows & (1u << o)) {  // wave-uniform
      const int64_t row = __builtin_amdgcn_readlane(my_row, o);
      const uint16_t* x = sd.rows + (row * a.hkv + h) * D;
#pragma unroll
      for (int k = 0; k < CPL; ++k) xv[o][k] = act_to_f32<BF16>(x[lane + 64 * k]);
    }
  }
  float ss[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    ss[k] = 0.0f;
#pragma unroll
    for (int o = 0; o < kBlock; ++o) ss[k] = __builtin_fmaf(xv[o][k], xv[o][k], ss[k]);  // +0 for absent rows
  }
  float r[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k) r[k] = __builtin_sqrtf(ss[k] / (float)n);
  uint32_t bytes[3];
  record_from_norms<D>(r, a.cap, bytes);
  if (lane == 0) {
    uint32_t* w = reinterpret_cast<uint32_t*>(rec);
    w[0] = bytes[0];
    w[1] = bytes[1];
    w[2] = bytes[2];
  }
}

// Per-sequence calibration, second launch: a block this call opens takes the outlier set
// of its leader row's sequence (the record bytes 0..11 of seq_records) instead of one
// computed from the call's rows. One thread per (row, head, K|V).
template <int D>
__global__ __launch_bounds__(256) void k_fp4_adopt(Fp4Args a) {
  using TL = Fp4Tile<D>;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)a.num_tokens * a.hkv) return;
  const int64_t i = idx / a.hkv, h = idx - i * a.hkv;
  const int64_t slot = a.slots[i];
  if (slot < 0 || slot >= a.nslots) return;
  const int64_t bh = (slot >> 4) * a.hkv + h;
  const int off = (int)(slot & 15);
  uint8_t* rec = a.side[blockIdx.z].tiles + bh * TL::kBytes + TL::kRecord;
  const uint32_t pending = ~*reinterpret_cast<const volatile uint32_t*>(rec + 12) & 0xFFFFu;
  if (!(pending & (1u << off)) || off != __builtin_ctz(pending)) return;  // not the leader
  const int32_t sq = a.token_seq[i];
  uint32_t w0 = 0xFFFFFF00u, w1 = 0xFFFFFFFFu, w2 = 0xFFFFFFFFu;  // no outliers
  if (sq < 0 || sq >= a.num_seqs) {
    flag(a.err, PA_DEVERR_BAD_CONTEXT);
  } else {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(
        a.seq_records + (((int64_t)sq * 2 + blockIdx.z) * a.hkv + h) * 16);
    w0 = src[0];
    w1 = src[1];
    w2 = src[2];
  }
  uint32_t* w = reinterpret_cast<uint32_t*>(rec);
  w[0] = w0;
  w[1] = w1;
  w[2] = w2;
}

// Per-sequence outlier sets: one workgroup (4 waves) per (sequence, head, K|V) sums the
// squares of the sequence's rows per channel (wave w takes rows w, w + 4, ...; the four
// partial sums are added in a fixed order), then wave 0 forms the record.
template <bool BF16, int D>
__global__ __launch_bounds__(256) void k_fp4_seq_outliers(SeqOutlierArgs a) {
  constexpr int CPL = D / 64;
  const int sq = blockIdx.x, h = blockIdx.y, side = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint16_t* rows = side ? a.v_rows : a.k_rows;
  const int64_t r0 = a.row_start[sq], r1 = a.row_start[sq + 1];
  const bool bad = r0 < 0 || r1 < r0 || r1 > a.num_rows;
  __shared__ float part[4][D];
  float ss[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k) ss[k] = 0.0f;
  if (!bad) {
    for (int64_t r = r0 + wave; r < r1; r += 4) {
      const uint16_t* x = rows + (r * a.hkv + h) * D;
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        const float v = act_to_f32<BF16>(x[lane + 64 * k]);
        ss[k] = __builtin_fmaf(v, v, ss[k]);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < CPL; ++k) part[wave][lane + 64 * k] = ss[k];
  __syncthreads();
  if (wave != 0) return;
  uint32_t* out = reinterpret_cast<uint32_t*>(a.records + (((int64_t)sq * 2 + side) * a.hkv + h) * 16);
  const int64_t n = bad ? 0 : r1 - r0;
  uint32_t bytes[3] = {0xFFFFFF00u, 0xFFFFFFFFu, 0xFFFFFFFFu};  // no outliers
  if (n > 0) {
    float r[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      const int c = lane + 64 * k;
      const float tot = ((part[0][c] + part[1][c]) + part[2][c]) + part[3][c];
      r[k] = __builtin_sqrtf(tot / (float)n);
    }
    record_from_norms<D>(r, a.cap, bytes);
  }
  if (lane == 0) {
    if (bad) flag(a.err, PA_DEVERR_BAD_CONTEXT);
    out[0] = bytes[0];
    out[1] = bytes[1];
    out[2] = bytes[2];
    out[3] = 0xFFFFFFFFu;
  }
}

// One wave per (row, head, K|V); lane l owns channels 2l and 2l + 1 (one packed byte).
template <bool BF16, int D>
__global__ __launch_bounds__(64 * kRowsPerWg) void k_fp4_encode(Fp4Args a) {
  using TL = Fp4Tile<D>;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = blockIdx.x * kRowsPerWg + wave;
  const int h = blockIdx.y;
  const bool vside = blockIdx.z == 1;
  const Fp4Side& sd = a.side[blockIdx.z];
  const int lane = threadIdx.x & 63;
  __shared__ int64_t wg_slot[kRowsPerWg];
  __shared__ uint32_t wg_bits[kRowsPerWg][64];

  int64_t slot = -1;  // -1: this wave stores nothing
  if (i < a.num_tokens) {
    slot = a.slots[i];
    if (slot >= a.nslots) slot = -1;
  }
  Fp4VBits vb;  // V: this lane's code word and its bits for this token
  if (slot >= 0) {
    const int64_t bh = (slot >> 4) * a.hkv + h;
    const int off = (int)(slot & 15);
    uint8_t* tile = sd.tiles + bh * TL::kBytes;
    uint8_t* rec = tile + TL::kRecord;
    const uint4 r4 = *reinterpret_cast<const uint4*>(rec);  // bytes 12..15 ignored
    const uint32_t rw[3] = {r4.x, r4.y, r4.z};
    int count = (int)(rw[0] & 0xFFu);
    if (count == 0xFF) {  // never calibrated: cannot happen after the calibrate launch
      if (lane == 0) flag(a.err, PA_DEVERR_UNCALIBRATED);
      slot = -1;
    } else {
      if (count > a.cap) count = a.cap;
      fp4_encode_row<BF16, D>(sd.rows + ((int64_t)i * a.hkv + h) * D, tile,
                              sd.out_val + bh * (a.cap - 1) * kBlock, off, vside, rw, count, vb);
    }
  }
  if (!vside) return;  // uniform over the workgroup

  // V codes of four tokens share each 32-bit word. When this workgroup's rows are a whole
  // aligned four of one block (the usual case in prefill), wave 0 stores the merged words;
  // otherwise other calls' or workgroups' rows may share the words, and each lane merges
  // its nibbles with atomics on disjoint bits (clear, then set).
  if (lane == 0) wg_slot[wave] = slot;
  wg_bits[wave][lane] = vb.bits;
  __syncthreads();
  const int64_t s0 = wg_slot[0];
  bool full = s0 >= 0 && (s0 & 3) == 0;
#pragma unroll
  for (int w = 1; w < kRowsPerWg; ++w) full = full && wg_slot[w] == s0 + w;
  if (full) {
    if (wave == 0 && vb.word) {
      uint32_t word = 0u;
#pragma unroll
      for (int w = 0; w < kRowsPerWg; ++w) word |= wg_bits[w][lane];
      *vb.word = word;
    }
  } else if (vb.word) {
    atomicAnd(vb.word, ~vb.mask);
    atomicOr(vb.word, vb.bits);
  }
}

// ---------------------------------------------------------------------------------
// FP8 per-head scale: fp32(absmax / 448). absmax via atomicMax on the fp32 bit pattern
// (non-negative floats order like their bit patterns).
// ---------------------------------------------------------------------------------
__global__ void k_scale_init(uint32_t* bits, int32_t hkv) {
  const int t = threadIdx.x;
  if (t < hkv) bits[t] = 0u;
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_absmax(const uint4* __restrict__ x, int64_t rows,
                                                int32_t hkv, int32_t chunks, uint32_t* bits) {
  const int h = blockIdx.y;
  float m = 0.0f;
  const int64_t n = rows * chunks;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = t / chunks, c = t - r * chunks;
    const uint4 v = x[(r * hkv + h) * chunks + c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      m = fmaxf(m, __builtin_fabsf(act_to_f32<BF16>(w[e] & 0xFFFFu)));
      m = fmaxf(m, __builtin_fabsf(act_to_f32<BF16>(w[e] >> 16)));
    }
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) atomicMax(bits + h, __float_as_uint(m));
}

__global__ void k_scale_finish(uint32_t* bits, int32_t hkv, float fmax) {
  const int t = threadIdx.x;
  if (t < hkv) {
    const float a = __uint_as_float(bits[t]);
    reinterpret_cast<float*>(bits)[t] = a / fmax;
  }
}

template <int D>
__global__ __launch_bounds__(256) void k_reset_records(uint8_t* tiles_k, uint8_t* tiles_v,
                                                       const int32_t* __restrict__ ids, int32_t n,
                                                       int32_t hkv, int32_t nb) {
  using TL = Fp4Tile<D>;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)n * hkv) return;
  const int32_t b = ids[t / hkv];
  if (b < 0 || b >= nb) return;
  const int64_t bh = (int64_t)b * hkv + t % hkv;
  const uint4 ff = make_uint4(~0u, ~0u, ~0u, ~0u);
  *reinterpret_cast<uint4*>(tiles_k + bh * TL::kBytes + TL::kRecord) = ff;
  *reinterpret_cast<uint4*>(tiles_v + bh * TL::kBytes + TL::kRecord) = ff;
}

// ---------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------
static inline unsigned grid1(int64_t n, int threads) { return (unsigned)((n + threads - 1) / threads); }

int launch_write(const pa_kv_pool& p, const void* k_new, const void* v_new, bool bf16,
                 int32_t T, const int64_t* slots, int32_t* err, hipStream_t st,
                 const int32_t* token_seq, const uint8_t* seq_records, int32_t num_seqs) {
  const int64_t nslots = (int64_t)p.num_blocks * kBlock;
  const int D = p.head_dim, hkv = p.num_kv_heads;
  if (T == 0) return PA_OK;
  if (p.dtype != PA_KV_FP4_E2M1_OUTL) {
    const bool fp8 = p.dtype != PA_KV_F16 && p.dtype != PA_KV_BF16;
    const bool e5 = p.dtype == PA_KV_FP8_E5M2 || p.dtype == PA_KV_FP8_E5M2_TOKEN;
    const bool tok = p.dtype == PA_KV_FP8_E4M3_TOKEN || p.dtype == PA_KV_FP8_E5M2_TOKEN;
    // threads per (token, head) row: 16-byte chunks of the copy, 16 values for FP8 (whose
    // threads take a window of four rows)
    const int ch = fp8 ? D / 16 : D * 2 / 16;
    const int64_t per_tok = (int64_t)hkv * ch;
    const int64_t row_u4 = (int64_t)hkv * D * 2 / 16;  // one input token row in 16 B units
    const int64_t max_tok = (((int64_t)1 << 31) / per_tok) & ~(int64_t)3;
    for (int64_t t0 = 0; t0 < T; t0 += max_tok) {
      const int32_t n = (int32_t)(T - t0 < max_tok ? T - t0 : max_tok);
      const uint4* kn = (const uint4*)k_new + t0 * row_u4;
      const uint4* vn = (const uint4*)v_new + t0 * row_u4;
      if (!fp8) {
        const dim3 g(grid1((int64_t)n * per_tok, 256));
        auto kern = D == 128 ? k_write_copy<16> : k_write_copy<8>;
        hipLaunchKernelGGL(kern, g, dim3(256), 0, st, kn, vn, (uint4*)p.k, (uint4*)p.v,
                           slots + t0, n, hkv, nslots, err);
      } else {
        const dim3 g(grid1((((int64_t)n + 3) / 4) * per_tok, 256));
        // kernel table: [token scales][bf16][D == 128][e5]
        void (*const tab[2][2][2][2])(const uint4*, const uint4*, uint8_t*, uint8_t*,
                                      const float*, const float*, const int64_t*, int32_t,
                                      int32_t, int64_t, int32_t*) = {
            {{{k_write_fp8<false, 4, false, false>, k_write_fp8<false, 4, true, false>},
              {k_write_fp8<false, 8, false, false>, k_write_fp8<false, 8, true, false>}},
             {{k_write_fp8<true, 4, false, false>, k_write_fp8<true, 4, true, false>},
              {k_write_fp8<true, 8, false, false>, k_write_fp8<true, 8, true, false>}}},
            {{{k_write_fp8<false, 4, false, true>, k_write_fp8<false, 4, true, true>},
              {k_write_fp8<false, 8, false, true>, k_write_fp8<false, 8, true, true>}},
             {{k_write_fp8<true, 4, false, true>, k_write_fp8<true, 4, true, true>},
              {k_write_fp8<true, 8, false, true>, k_write_fp8<true, 8, true, true>}}}};
        hipLaunchKernelGGL(tab[tok][bf16][D == 128][e5], g, dim3(256), 0, st, kn, vn,
                           (uint8_t*)p.k, (uint8_t*)p.v, p.k_scale, p.v_scale, slots + t0, n,
                           hkv, nslots, err);
      }
    }
  } else {
    // heads index grid.y
    if ((D != 64 && D != 128) || hkv > 65535) return PA_ERR_SHAPE;
    Fp4Args a;
    a.side[0] = {(const uint16_t*)k_new, (uint8_t*)p.k, p.k_out_val};
    a.side[1] = {(const uint16_t*)v_new, (uint8_t*)p.v, p.v_out_val};
    a.slots = slots;
    a.num_tokens = T;
    a.hkv = hkv;
    a.head_dim = D;
    a.cap = outlier_capacity(D);
    a.nslots = nslots;
    a.err = err;
    a.token_seq = token_seq;
    a.seq_records = seq_records;
    a.num_seqs = num_seqs;
    const dim3 gt(grid1((int64_t)T * hkv, 256), 1, 2);
    const dim3 g((unsigned)((T + kRowsPerWg - 1) / kRowsPerWg), hkv, 2);
    const bool d128 = D == 128;
    hipLaunchKernelGGL(d128 ? k_fp4_mark<128> : k_fp4_mark<64>, gt, dim3(256), 0, st, a);
    if (seq_records) {
      hipLaunchKernelGGL(d128 ? k_fp4_adopt<128> : k_fp4_adopt<64>, gt, dim3(256), 0, st, a);
    } else {
      auto cal = d128 ? (bf16 ? k_fp4_calibrate<true, 128> : k_fp4_calibrate<false, 128>)
                      : (bf16 ? k_fp4_calibrate<true, 64> : k_fp4_calibrate<false, 64>);
      hipLaunchKernelGGL(cal, g, dim3(64 * kRowsPerWg), 0, st, a);
    }
    auto enc = d128 ? (bf16 ? k_fp4_encode<true, 128> : k_fp4_encode<false, 128>)
                    : (bf16 ? k_fp4_encode<true, 64> : k_fp4_encode<false, 64>);
    hipLaunchKernelGGL(enc, g, dim3(64 * kRowsPerWg), 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int launch_fp4_seq_outliers(const void* k_rows, const void* v_rows, bool bf16, int64_t num_rows,
                           int32_t hkv, int32_t D, const int32_t* row_start, int32_t num_seqs,
                           uint8_t* records, int32_t* err, hipStream_t st) {
  if (D != 64 && D != 128) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  SeqOutlierArgs a;
  a.k_rows = (const uint16_t*)k_rows;
  a.v_rows = (const uint16_t*)v_rows;
  a.row_start = row_start;
  a.num_rows = num_rows;
  a.hkv = hkv;
  a.cap = outlier_capacity(D);
  a.records = records;
  a.err = err;
  auto kern = D == 128 ? (bf16 ? k_fp4_seq_outliers<true, 128> : k_fp4_seq_outliers<false, 128>)
                       : (bf16 ? k_fp4_seq_outliers<true, 64> : k_fp4_seq_outliers<false, 64>);
  hipLaunchKernelGGL(kern, dim3((unsigned)num_seqs, hkv, 2), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int launch_fp8_scales(const void* x, bool bf16, bool e5m2, int64_t rows, int32_t hkv, int32_t D,
                      float* scale_out, hipStream_t st) {
  uint32_t* bits = reinterpret_cast<uint32_t*>(scale_out);
  hipLaunchKernelGGL(k_scale_init, dim3(1), dim3(256), 0, st, bits, hkv);
  if (rows > 0) {
    const int chunks = D / 8;
    const int64_t n = rows * chunks;
    unsigned gx = grid1(n, 256);
    if (gx > 1024) gx = 1024;
    auto kern = bf16 ? k_absmax<true> : k_absmax<false>;
    hipLaunchKernelGGL(kern, dim3(gx, hkv), dim3(256), 0, st, (const uint4*)x, rows, hkv, chunks,
                       bits);
  }
  hipLaunchKernelGGL(k_scale_finish, dim3(1), dim3(256), 0, st, bits, hkv,
                     e5m2 ? 57344.0f : 448.0f);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int launch_reset(const pa_kv_pool& p, const int32_t* ids, int32_t n, hipStream_t st) {
  if (n == 0) return PA_OK;
  const int64_t total = (int64_t)n * p.num_kv_heads;
  if (p.head_dim != 64 && p.head_dim != 128) return PA_ERR_SHAPE;
  hipLaunchKernelGGL(p.head_dim == 128 ? k_reset_records<128> : k_reset_records<64>,
                     dim3(grid1(total, 256)), dim3(256), 0, st,
                     (uint8_t*)p.k, (uint8_t*)p.v, ids, n, p.num_kv_heads, p.num_blocks);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace pa
