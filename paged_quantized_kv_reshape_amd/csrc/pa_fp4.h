// pa_fp4.h - the 4-bit format's per-row pieces (internal to libpa): the tile regions, the
// outlier set from channel norms and the encode of one row, shared by the write kernels
// and the decode that appends each sequence's new token itself (dailyaiworld.com, "vLLM
// 0.7 Ships Unified KV Cache Compression", "Technical Breakdown: Dynamic Quantization with
// Outlier Retention", steps 1-3).
#pragma once

#include "../../include/pa.h"
#include "pa_device.h"

namespace pa {

// Regions of one (block, head) FP4 tile.
template <int D>
struct Fp4Tile {
  static constexpr int kBytes = PA_FP4_TILE_BYTES(D);
  static constexpr int kScale = PA_FP4_SCALE_OFF(D);
  static constexpr int kRecord = PA_FP4_RECORD_OFF(D);
  static constexpr int kSlot0 = PA_FP4_SLOT0_OFF(D);
  static_assert(kScale % 16 == 0 && kRecord % 16 == 0 && kSlot0 % 8 == 0, "FP4 tile layout");
};
// The outlier set from per-channel RMS norms r (channel lane + 64 k in r[k]) of one wave:
// mu and population sigma over the D norms, channels with r >= mu + 3.2 sigma (none when
// sigma = 0), ascending, at most cap of them; returned as record bytes 0..11 (count, ids,
// 0xFF padding) in three words.
template <int D>
__device__ __forceinline__ void record_from_norms(const float (&r)[D / 64], int cap,
                                                  uint32_t (&bytes)[3]) {
  constexpr int CPL = D / 64;
  float part = 0.0f;
#pragma unroll
  for (int k = 0; k < CPL; ++k) part += r[k];
  const float mu = wave_sum(part) / (float)D;
  float dev = 0.0f;
#pragma unroll
  for (int k = 0; k < CPL; ++k) dev += (r[k] - mu) * (r[k] - mu);
  const float sigma = __builtin_sqrtf(wave_sum(dev) / (float)D);
  const float thr = mu + kOutlierSigmas * sigma;
  bytes[0] = bytes[1] = bytes[2] = 0xFFFFFFFFu;
  int count = 0;
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const bool hit = sigma != 0.0f && r[k] >= thr;
    uint64_t mask = __ballot(hit);
    while (mask) {
      const int c = __builtin_ctzll(mask) + 64 * k;
      mask &= mask - 1;
      if (count < cap) {
        const int pos = 1 + count;  // byte position in the record
        bytes[pos >> 2] &= ~(0xFFu << ((pos & 3) * 8));
        bytes[pos >> 2] |= (uint32_t)c << ((pos & 3) * 8);
      }
      ++count;
    }
  }
  const int stored = count < cap ? count : cap;
  bytes[0] = (bytes[0] & ~0xFFu) | (uint32_t)stored;
}

// One FP4 row, calibrated alone (its block's first write holds only this row): the norm of
// channel c is sqrt(fp32(x_c^2) / 1), as the calibrate kernel computes it for one row.
template <bool BF16, int D>
__device__ __forceinline__ void fp4_calibrate_row(const uint16_t* row, int cap,
                                                  uint32_t (&bytes)[3]) {
  constexpr int CPL = D / 64;
  const int lane = threadIdx.x & 63;
  float r[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const float x = act_to_f32<BF16>(row[lane + 64 * k]);
    r[k] = __builtin_sqrtf(__builtin_fmaf(x, x, 0.0f) / 1.0f);
  }
  record_from_norms<D>(r, cap, bytes);
}

// V codes of four tokens share each 32-bit word: the word, bits and mask of this lane's
// two nibbles of one row (word null: nothing to store).
struct Fp4VBits {
  uint32_t* word = nullptr;
  uint32_t bits = 0u, mask = 0u;
};

// One wave encodes one row (one token of one kv head, K or V) with its block's record
// words rw (count already at most the capacity): per-token scale fp32(inlier absmax / 6),
// E2M1 codes of the inliers, +0 codes at the outlier channels, whose fp16 values go to
// slot 0 of the tile (first outlier) and to out_val_bh[(j - 1) * 16 + off] (the others).
// K codes are stored here; V codes are returned in vb for the caller to merge. Lane 0
// stores the scale and sets the record's bytes 12..15 back to 0xFF.
template <bool BF16, int D>
__device__ __forceinline__ void fp4_encode_row(const uint16_t* row, uint8_t* tile,
                                               uint16_t* out_val_bh, int off, bool vside,
                                               const uint32_t (&rw)[3], int count,
                                               Fp4VBits& vb) {
  using TL = Fp4Tile<D>;
  const int lane = threadIdx.x & 63;
  uint8_t* rec = tile + TL::kRecord;
  const bool active = lane < D / 2;
  const int c0 = 2 * lane, c1 = c0 + 1;
  float x0 = 0.0f, x1 = 0.0f;
  if (active) {
    const uint32_t pair = *reinterpret_cast<const uint32_t*>(row + c0);
    x0 = act_to_f32<BF16>(pair & 0xFFFFu);
    x1 = act_to_f32<BF16>(pair >> 16);
  }
  bool out0 = false, out1 = false;
  for (int j = 0; j < count; ++j) {
    const int pos = 1 + j;
    const int c = (int)((rw[pos >> 2] >> ((pos & 3) * 8)) & 0xFFu);
    out0 |= (c == c0);
    out1 |= (c == c1);
  }
  const float a0 = (active && !out0) ? __builtin_fabsf(x0) : 0.0f;
  const float a1 = (active && !out1) ? __builtin_fabsf(x1) : 0.0f;
  const float amax = wave_max(fmaxf(a0, a1));
  const float sc = amax / 6.0f;
  uint32_t q0 = 0u, q1 = 0u;
  if (sc != 0.0f) {
    q0 = out0 ? 0u : encode_e2m1(x0 / sc);
    q1 = out1 ? 0u : encode_e2m1(x1 / sc);
  }
  if (active) {
    if (!vside) {
      tile[off * (D / 2) + lane] = (uint8_t)(q0 | (q1 << 4));  // K: token rows
    } else {
      // V: a chunk holds D / 16 channels of four tokens in D / 32 words, two channels per
      // word; channels 2 lane and 2 lane + 1 sit in word lane % WPC of chunk
      // (lane / WPC) * 4 + off / 4, at bit 8 ((off % 4) / 2) + 4 (off % 2) and 16 above
      constexpr int WPC = D / 32;
      const int sh = 8 * ((off & 3) >> 1) + 4 * (off & 1);
      vb.word = reinterpret_cast<uint32_t*>(tile) +
                (((lane / WPC) * 4 + (off >> 2)) * WPC + (lane % WPC));
      vb.bits = (q0 << sh) | (q1 << (sh + 16));
      vb.mask = (0xFu << sh) | (0xFu << (sh + 16));
    }
  }
  for (int j = 0; j < count; ++j) {
    const int pos = 1 + j;
    const int c = (int)((rw[pos >> 2] >> ((pos & 3) * 8)) & 0xFFu);
    if (active && (c >> 1) == lane) {
      const float xv = (c & 1) ? x1 : x0;
      const uint16_t hv = bitcast<uint16_t>((_Float16)xv);
      if (j == 0)
        reinterpret_cast<uint16_t*>(tile + TL::kSlot0)[off] = hv;
      else
        out_val_bh[(j - 1) * kBlock + off] = hv;
    }
  }
  if (lane == 0) {
    reinterpret_cast<float*>(tile + TL::kScale)[off] = sc;
    *reinterpret_cast<uint32_t*>(rec + 12) = 0xFFFFFFFFu;
  }
}

}  // namespace pa
