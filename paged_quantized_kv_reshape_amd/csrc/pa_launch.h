// pa_launch.h - host-side launch entry points of the gfx950 kernels (internal to libpa).
// The C ABI in pa_api.cpp validates arguments and then calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pa.h"

namespace pa {

// floor(D / (1 + 3.2^2)): the most channels that can sit at or above mean + 3.2 sigma.
inline int outlier_capacity(int head_dim) {
  return head_dim == 128 ? 11 : head_dim == 64 ? 5 : -1;
}

// token_seq / seq_records / num_seqs: FP4 per-sequence calibration (blocks the call opens
// take their sequence's outlier set); nullptr / 0 for the per-block calibration.
int launch_write(const pa_kv_pool& p, const void* k_new, const void* v_new, bool bf16, int32_t T,
                 const int64_t* slots, int32_t* err, hipStream_t st,
                 const int32_t* token_seq = nullptr, const uint8_t* seq_records = nullptr,
                 int32_t num_seqs = 0);
int launch_fp4_seq_outliers(const void* k_rows, const void* v_rows, bool bf16, int64_t num_rows,
                           int32_t hkv, int32_t D, const int32_t* row_start, int32_t num_seqs,
                           uint8_t* records, int32_t* err, hipStream_t st);
int launch_fp8_scales(const void* x, bool bf16, bool e5m2, int64_t rows, int32_t hkv, int32_t D,
                      float* scale_out, hipStream_t st);
int launch_reset(const pa_kv_pool& p, const int32_t* ids, int32_t n, hipStream_t st);

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const uint16_t* k_out_val;  // FP4 outlier slots 1 .. cap - 1
  const uint16_t* v_out_val;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* out;       // [S, Hq, D] when partition_size == 0
  float* part_out;  // [S, Hq, P, D] otherwise
  float* part_lse;  // [S, Hq, P]
  int32_t* err;
  // decode with append (pa_append_decode[_n]): sequence s's new_tokens new K/V rows
  // [new_tokens][Hkv][D] at k_new / v_new + s * new_tokens * Hkv * D (activation dtype of
  // q), written at positions L_s - new_tokens .. L_s - 1 first
  const void* k_new;
  const void* v_new;
  int32_t new_tokens;
  uint32_t* sink;              // gather probe: [1024] XOR words
  const int32_t* query_start;  // multi-token queries: [S + 1] row offsets of q and out
  int32_t max_query_len, num_queries;
  int32_t num_seqs, num_q_heads, num_kv_heads, group, num_blocks, max_blocks, partition_size,
      max_partitions, cap;
  float sm_scale_log2;  // sm_scale * log2(e)
};

int launch_decode(const DecodeArgs& a, int kv_dtype, bool q_bf16, int head_dim, int waves,
                  hipStream_t st);
// gather-only ceiling (pa_gather_probe): the decode's launch and loads, no arithmetic
int launch_gather_probe(const DecodeArgs& a, int kv_dtype, int head_dim, int waves,
                        uint32_t* sink, hipStream_t st);
// multi-token queries (pa_prefill): the paired-block kernel, every pool format;
// col_tiles 2 or 3 fixes the column tiles per wave (0: the format's default)
int launch_prefill(const DecodeArgs& a, int kv_dtype, bool q_bf16, int head_dim, int col_tiles,
                   hipStream_t st);

// Whole-block copy: array j of the pool has vecs_per_block[j] 16-byte vectors per block.
struct CopyArgs {
  const void* src[4];
  void* dst[4];
  uint32_t vecs_per_block[4];
  const int32_t* pairs;  // [num_pairs][2] (source, destination)
  int32_t num_pairs, num_arrays, src_blocks, dst_blocks;
  int32_t* err;
  bool streaming;  // non-temporal loads and stores (copies within one device pool)
};
int launch_copy_blocks(const CopyArgs& a, hipStream_t st);

int launch_merge(const float* part_out, const float* part_lse, const int32_t* context_lens,
                 int32_t S, int32_t Hq, int32_t D, int32_t P, int32_t ps, float* out,
                 float* lse_out, hipStream_t st);

}  // namespace pa
