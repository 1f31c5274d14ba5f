/*
 * pa.h - C ABI of the paged, quantized KV-cache library for AMD Instinct MI355X (gfx950).
 *
 * Two operations make up the hot path of paged decode over a low-precision KV cache:
 *
 *   cache write  - scatter each new token's K/V row into its slot of a fixed 16-token
 *                  physical block, quantizing on the fly (dailyaiworld.com, "vLLM 0.7 Ships
 *                  Unified KV Cache Compression": the engine diagram and the section "The KV
 *                  Cache Memory Crisis in Enterprise Agent Deployments"; xonoai.com field
 *                  report on vLLM v0.7.2, "Deconstructing the v0.7.2 Architecture").
 *   paged decode - gather a sequence's blocks through its block table, dequantize, and run
 *                  softmax attention for one new query token, optionally split into
 *                  context partitions that a log-sum-exp merge recombines (inferensys
 *                  glossary "vLLM", PagedAttention entry; dailyaiworld.com, "Technical
 *                  Breakdown: Dynamic Quantization with Outlier Retention", step 4).
 *
 * Conventions shared by every entry point
 *   - Pointers are device pointers unless stated otherwise. The caller owns all memory;
 *     the library allocates no device memory and keeps no mutable global state, so calls
 *     from several host threads or streams are safe if their buffers do not overlap. (The
 *     host-side block allocator below is an object the caller creates and destroys.)
 *   - Arguments are validated on the host before anything is launched; a failed check
 *     returns a negative pa_status and launches nothing. Work is queued asynchronously
 *     on `stream` (a hipStream_t; NULL = the default stream). Device-side faults surface
 *     at the caller's next synchronization.
 *   - Device-side checks (a block id outside [0, num_blocks), a slot outside
 *     [0, num_blocks * 16), a context length outside [1, max_blocks_per_seq * 16), a read
 *     of an FP4 block that was never written) skip the offending access and OR a bit into
 *     the optional `dev_err` word (an int32 in device memory the caller zeroes; NULL = no
 *     reporting). Bits: PA_DEVERR_*.
 *   - All arrays are dense, row-major, in the shapes written below, 16-byte aligned.
 *   - Query head h reads kv head h / (num_q_heads / num_kv_heads) (grouped-query attention
 *     with contiguous groups); num_q_heads / num_kv_heads must be 1..16.
 *   - head_dim is 64 or 128 in every format; block_size is 16 (the block size the pages use: xonoai.com
 *     report, "Deconstructing the v0.7.2 Architecture", and its --block-size 16 flag).
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_BLOCK_SIZE 16

/* KV cache storage formats (the --kv-cache-dtype choices on the pages, plus 16-bit). */
typedef enum {
  PA_KV_F16 = 0,            /* fp16 copy, no quantization                              */
  PA_KV_BF16 = 1,           /* bf16 copy, no quantization                              */
  PA_KV_FP8_E4M3 = 2,       /* OCP E4M3FN codes, one fp32 scale per kv head (K and V)  */
  PA_KV_FP4_E2M1_OUTL = 3,  /* E2M1 codes + per-token fp32 scale + fp16 outlier buffer */
  PA_KV_FP8_E5M2 = 4,       /* OCP E5M2 codes, one fp32 scale per kv head (K and V)    */
  PA_KV_FP8_E4M3_TOKEN = 5, /* E4M3FN codes + a per-token fp32 scale set at write time */
  PA_KV_FP8_E5M2_TOKEN = 6  /* E5M2 codes + a per-token fp32 scale set at write time   */
} pa_kv_dtype;

/* Activation (query and new K/V row) dtypes. */
typedef enum { PA_ACT_F16 = 0, PA_ACT_BF16 = 1 } pa_act_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL                                 */
  PA_ERR_SHAPE = -2,       /* a size is out of range or inconsistent                     */
  PA_ERR_DTYPE = -3,       /* unknown dtype or an unsupported kv/activation combination  */
  PA_ERR_BLOCK_SIZE = -4,  /* block_size != 16                                          */
  PA_ERR_CONTEXT = -5,     /* max_blocks_per_seq out of range                           */
  PA_ERR_PARTITION = -6,   /* partition_size not 0 and not a positive multiple of 16    */
  PA_ERR_LAUNCH = -7,      /* the HIP runtime refused a launch                          */
  PA_ERR_ALIGN = -8,       /* a pointer is not 16-byte aligned                          */
  PA_ERR_MEMORY = -9,      /* a pointer is not memory this GPU can access               */
  PA_ERR_EXHAUSTED = -10,  /* the block allocator has fewer free blocks than requested  */
  PA_ERR_STATE = -11,      /* the block allocator was asked about a block not in use    */
  PA_ERR_SCRATCH = -12,    /* the call needs more than the library's static scratch      */
  PA_ERR_SCALE = -13       /* sm_scale is not a positive finite number                   */
} pa_status;

#define PA_DEVERR_BAD_BLOCK 1        /* block table / copy pair id outside its pool: the
                                        attention calls skip that block's keys and values */
#define PA_DEVERR_BAD_SLOT 2         /* slot_mapping entry outside [0, num_blocks * 16)   */
#define PA_DEVERR_BAD_CONTEXT 4      /* context_lens entry outside [1, MB * 16]           */
#define PA_DEVERR_UNCALIBRATED 8     /* decode read an FP4 block whose record is unset    */

/*
 * The paged KV pool (passed by host pointer; the arrays it points to are device memory).
 *
 *   PA_KV_F16 / PA_KV_BF16 : k, v   [num_blocks, num_kv_heads, 16, head_dim] 16-bit values
 *   PA_KV_FP8_E4M3 / _E5M2 : k      [num_blocks, num_kv_heads, 16, head_dim] uint8 codes
 *                            v      [num_blocks, num_kv_heads, 16 * head_dim] uint8 codes,
 *                                   stored by channel: token t, channel ch of a (block,
 *                                   kv head) run at byte PA_FP8_V_BYTE(t, ch, head_dim)
 *                            k_scale, v_scale [num_kv_heads] fp32 (inputs, read-only):
 *                            the stored value is code * scale (per layer and kv head;
 *                            see pa_fp8_head_scales). Both OCP FP8 formats are the pages'
 *                            ("FP8 (E4M3 and E5M2)", xonoai.com field report,
 *                            "Deconstructing the v0.7.2 Architecture").
 *   PA_KV_FP8_E4M3_TOKEN / _E5M2_TOKEN :
 *                            k  [num_blocks, num_kv_heads, PA_FP8T_TILE_BYTES(head_dim)]
 *                               bytes, one run per (block, kv head): codes
 *                               [16 tokens][head_dim], then at PA_FP8T_SCALE_OFF the 16
 *                               per-token fp32 scales of K and at PA_FP8T_VSCALE_OFF the
 *                               16 of V (together one whole 128-byte line);
 *                            v  [num_blocks, num_kv_heads, PA_FP8T_VTILE_BYTES(head_dim)]
 *                               bytes: the V codes only, by channel as above.
 *                            The scale of a token row is fp32(max |x| / 448) (E4M3) or
 *                            fp32(max |x| / 57344) (E5M2), set when the row is written:
 *                            quantization on the fly (dailyaiworld.com, "vLLM 0.7 Ships
 *                            Unified KV Cache Compression", opening section), with no
 *                            per-head calibration to drift (xonoai.com report, closing
 *                            section). No scale arrays are needed.
 *   PA_KV_FP4_E2M1_OUTL    : k, v   [num_blocks, num_kv_heads, PA_FP4_TILE_BYTES(head_dim)]
 *                                   bytes: one contiguous run per (block, kv head) holding
 *                                   everything a decode reads for that block, so it is
 *                                   fetched in whole 128-byte lines:
 *                            [0, 8 D)       E2M1 codes, 4 bits each. K: token rows
 *                                           [16][D/2], even channel in the low nibble.
 *                                           V: chunks of NC = D / 16 channels of four
 *                                           tokens (2 NC bytes: 16 at D = 128, 8 at
 *                                           D = 64); chunk (ch / NC) * 4 + t / 4 holds
 *                                           channels NC g .. NC g + NC - 1 of tokens
 *                                           4 j .. 4 j + 3; in it byte 2 (ch % NC) holds
 *                                           tokens 4 j, 4 j + 1 and the next byte tokens
 *                                           4 j + 2, 4 j + 3 of channel ch, the even
 *                                           token in the low nibble (a decode lane reads
 *                                           one chunk and converts token pairs).
 *                            PA_FP4_SCALE_OFF   16 per-token fp32 scales (value = code *
 *                                               scale for the inlier channels)
 *                            PA_FP4_RECORD_OFF  16-byte outlier record: byte 0 = outlier
 *                                               count, or 0xFF while the block has never
 *                                               been written; bytes 1..count = ascending
 *                                               channel indices; the other bytes 0xFF
 *                            PA_FP4_SLOT0_OFF   fp16 bits of the first outlier channel's
 *                                               value, one per token (16 x 2 bytes)
 *                            then padding to a multiple of 128 bytes.
 *                            *_out_val [num_blocks, num_kv_heads, CAP - 1, 16] fp16 bits:
 *                                      slot j holds the (j + 1)-th outlier channel's value
 *                                      for each token offset; CAP = pa_outlier_capacity(D).
 *                            Every block's record must read 0xFF before the block is first
 *                            written: call pa_reset_blocks on new and on reused blocks.
 *   Fields a format does not use are ignored (may be NULL).
 */
#define PA_FP4_SCALE_OFF(head_dim) (8 * (head_dim))
#define PA_FP4_RECORD_OFF(head_dim) (8 * (head_dim) + 64)
#define PA_FP4_SLOT0_OFF(head_dim) (8 * (head_dim) + 80)
#define PA_FP4_TILE_BYTES(head_dim) ((8 * (head_dim) + 112 + 127) / 128 * 128)
/* FP8 V code runs (both scale kinds) by channel: with nt = head_dim / 16, channel ch is
 * channel j = ch % nt of group g = ch / nt. The run is head_dim / 64 pieces of 1024 bytes;
 * piece j / 4 is 64 slots of 16 bytes, slot 16 (t / 4) + g holding channels j = 4 (j / 4)
 * .. + 3 of group g for tokens 4 (t / 4) .. + 3, channel after channel, a channel's four
 * token bytes side by side. One 16-byte slot is what one lane of the P.V product takes for
 * its four keys, so a tile of V is loaded in whole lines with no byte shuffling. */
#define PA_FP8_V_BYTE(t, ch, head_dim)                                                   \
  ((((ch) % ((head_dim) / 16)) / 4) * 1024 +                                           \
   (16 * ((t) / 4) + (ch) / ((head_dim) / 16)) * 16 + (((ch) % ((head_dim) / 16)) % 4) * 4 + \
   (t) % 4)

/* per-token-scaled FP8 runs: K codes, K token scales, V token scales (k array); V codes
 * (v array). Every run is a whole number of 128-byte lines with no padding. */
#define PA_FP8T_SCALE_OFF(head_dim) (16 * (head_dim))
#define PA_FP8T_VSCALE_OFF(head_dim) (16 * (head_dim) + 64)
#define PA_FP8T_TILE_BYTES(head_dim) (16 * (head_dim) + 128)
#define PA_FP8T_VTILE_BYTES(head_dim) (16 * (head_dim))

typedef struct pa_kv_pool {
  int32_t dtype;          /* pa_kv_dtype */
  int32_t num_blocks;
  int32_t block_size;     /* must be 16 */
  int32_t num_kv_heads;
  int32_t head_dim;       /* 64 or 128 */
  int32_t reserved;
  void* k;
  void* v;
  uint16_t* k_out_val;    /* FP4 only */
  uint16_t* v_out_val;    /* FP4 only */
  const float* k_scale;   /* FP8 only */
  const float* v_scale;   /* FP8 only */
} pa_kv_pool;

/*
 * Host-only. Byte sizes of the pool arrays for a format, in the order
 * {k, v, k_out_val, v_out_val} (0 for arrays the format does not use). Returns PA_OK or an
 * error status.
 */
int pa_pool_layout(int32_t dtype, int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                   size_t bytes_out[4]);

/*
 * Host-only. Outlier slots per (block, kv head) of the FP4 format: the largest number of
 * channels whose per-channel RMS can reach mean + 3.2 sigma of head_dim values,
 * floor(head_dim / (1 + 3.2^2)) = 11 for 128, 5 for 64 (the threshold is the pages':
 * dailyaiworld.com, "Technical Breakdown: Dynamic Quantization with Outlier Retention",
 * step 2). Returns -PA_ERR_SHAPE-style negative status for an unsupported head_dim.
 */
int pa_outlier_capacity(int32_t head_dim);

/*
 * Cache write ("reshape and cache"). Row i of k_new / v_new [num_tokens, num_kv_heads,
 * head_dim] (activation dtype `act`) is stored at slot_mapping[i] = block * 16 + offset
 * (int64; negative = skip the row). Slots within one call must be distinct.
 *   F16 / BF16 : bit copy; the pool dtype must equal `act`.
 *   FP8        : code = E4M3(fp32(x / scale_h)), the correctly rounded fp32 quotient
 *                rounded to the nearest E4M3FN value, ties to even, saturating at +-448,
 *                sign of zero kept; scale 0 stores +0.
 *   FP4        : dailyaiworld.com, "Technical Breakdown: Dynamic Quantization with
 *                Outlier Retention", steps 1-3. A block whose record is 0xFF is calibrated
 *                by this call, separately per kv head and for K and V, on the rows of this
 *                call that land in it: per-channel RMS r_c over those rows, mean mu and
 *                population std sigma of the head_dim values r_c, outliers = channels with
 *                r_c >= mu + 3.2 sigma (none if sigma = 0), stored ascending in the record.
 *                Later writes reuse the record. Every row then stores fp16(x_c) for its
 *                block's outlier channels, code +0 at those channels, a scale
 *                s = fp32(max inlier |x_c| / 6) and codes E2M1(fp32(x_c / s)) (nearest,
 *                ties to even, saturating at +-6; s = 0 stores +0 codes).
 * Asynchronous on `stream`. Returns PA_OK or an error status (nothing launched on error).
 */
int pa_cache_write(const pa_kv_pool* pool, const void* k_new, const void* v_new, int32_t act,
                   int32_t num_tokens, const int64_t* slot_mapping, int32_t* dev_err,
                   void* stream);

/*
 * Per-kv-head FP8 scale of a tensor x [num_rows, num_kv_heads, head_dim] (activation dtype
 * `act`) for a pool of dtype kv_dtype (PA_KV_FP8_E4M3 or PA_KV_FP8_E5M2):
 * scale_out[h] = fp32(max |x[:, h, :]| / M), M = 448 (E4M3) or 57344 (E5M2), the
 * per-(layer, kv head) fp32 scale that maps each head's largest magnitude onto the
 * format's largest value (xonoai.com report, "Deconstructing the v0.7.2 Architecture" and
 * "Field Observations", on FP8 calibration). scale_out [num_kv_heads] fp32 is overwritten.
 * Call once for K and once for V. Asynchronous on `stream`.
 */
int pa_fp8_head_scales(const void* x, int32_t act, int32_t kv_dtype, int64_t num_rows,
                       int32_t num_kv_heads, int32_t head_dim, float* scale_out, void* stream);

/*
 * FP4 per-sequence calibration, the pages' wording taken literally: the per-channel norms
 * of the key and value vectors a sequence's prefill produces decide its outlier channels
 * (dailyaiworld.com, "Technical Breakdown: Dynamic Quantization with Outlier Retention",
 * steps 1-2), here once per (sequence, kv head, K|V) instead of once per block.
 *   k_rows, v_rows [num_rows, num_kv_heads, head_dim], activation dtype `act`: the rows
 *                 the sets come from (typically each sequence's first prefill chunk);
 *                 sequence s owns rows row_start[s] .. row_start[s + 1] - 1
 *   row_start     [num_seqs + 1] int32
 *   seq_records   [num_seqs, 2, num_kv_heads, 16] uint8 (written): K (index 0) and V (1)
 *                 sets in the block record format (count, ascending channel ids, 0xFF)
 * Same statistics as the per-block calibration: per-channel RMS over the rows, channels at
 * or above mean + 3.2 population sigma of the head_dim norms. head_dim 64 or 128. A sequence with
 * no rows gets an empty set; one whose range is not inside [0, num_rows) too, flagged
 * PA_DEVERR_BAD_CONTEXT. Asynchronous on `stream`.
 */
int pa_fp4_sequence_outliers(const void* k_rows, const void* v_rows, int32_t act,
                             int64_t num_rows, int32_t num_kv_heads, int32_t head_dim,
                             const int32_t* row_start, int32_t num_seqs, uint8_t* seq_records,
                             int32_t* dev_err, void* stream);

/*
 * pa_cache_write into an FP4 pool with per-sequence calibration: a block the call opens
 * takes the outlier set of its sequence from seq_records (pa_fp4_sequence_outliers) rather
 * than one computed from the call's rows in it, so a decode token that starts a block
 * encodes with the sequence's set. The sequence of a block is that of its lowest-offset
 * row in the call; blocks already written keep their set. token_seq [num_tokens] int32:
 * the sequence of each row; a row naming a sequence outside [0, num_seqs) opens its block
 * with no outliers and is flagged (PA_DEVERR_BAD_CONTEXT). The pool must be
 * PA_KV_FP4_E2M1_OUTL. Everything else as pa_cache_write. Asynchronous on `stream`.
 */
int pa_cache_write_seq_outliers(const pa_kv_pool* pool, const void* k_new, const void* v_new,
                                int32_t act, int32_t num_tokens, const int64_t* slot_mapping,
                                const int32_t* token_seq, const uint8_t* seq_records,
                                int32_t num_seqs, int32_t* dev_err, void* stream);

/*
 * Mark the listed physical blocks as never written (FP4 records set to 0xFF), so the next
 * write into each one calibrates it afresh: call it once for every block of a new pool,
 * and when the engine hands a freed block to a new sequence (inferensys glossary "vLLM", continuous batching entry: finished
 * sequences release their blocks to the pool). block_ids [n] int32, device memory.
 * No-op (PA_OK) for formats without records.
 */
int pa_reset_blocks(const pa_kv_pool* pool, const int32_t* block_ids, int32_t n, void* stream);

/*
 * Copy whole physical blocks from pool `src` to pool `dst`: for i < num_pairs, block
 * pairs[2 i + 1] of dst becomes a byte-for-byte copy of block pairs[2 i] of src in every
 * array the format uses (codes, the per-token scales and FP4 records inside the runs, the
 * FP4 outlier slots). Per-head FP8 scales are not block data and are not touched.
 *   - Copy on write: src == dst duplicates a block that several sequences share before
 *     one of them extends it (inferensys glossary "vLLM", PagedAttention entry: blocks
 *     shared across sequences for beam search, parallel sampling and prefix caching).
 *   - Swap: a second pool of the same format whose arrays are pinned host memory
 *     (hipHostMalloc) holds a preempted sequence's blocks; copying device -> host swaps
 *     them out, host -> device back in (inferensys glossary "vLLM", preemption by
 *     swapping KV blocks to CPU RAM, and CPU offloading). The GPU reads and writes the
 *     host pool in place.
 * The two pools must have the same dtype, num_kv_heads and head_dim (num_blocks may
 * differ; k_scale / v_scale are ignored). pairs [num_pairs][2] int32 (source, destination),
 * 8-byte aligned. Every pool array, pairs and dev_err must be device memory of the current
 * GPU or pinned host memory. When the pools' arrays differ (a swap) each pointer is looked
 * up first and anything else (pageable host memory) returns PA_ERR_MEMORY before any
 * launch; within one pool nothing is looked up (a few microseconds saved per call). Destinations must be distinct and, within one pool, not also sources
 * in the same call; otherwise the bytes of the affected blocks are unspecified (every
 * access still stays inside the pools). A pair naming a block outside its pool is skipped
 * and flagged (PA_DEVERR_BAD_BLOCK). A copied FP4 block keeps its calibration record, so
 * writes into the copy reuse the source's outlier set. Asynchronous on `stream`.
 */
int pa_copy_blocks(const pa_kv_pool* src, const pa_kv_pool* dst, const int32_t* pairs,
                   int32_t num_pairs, int32_t* dev_err, void* stream);

/*
 * Host-only reference-counted allocator of a pool's physical block ids (inferensys
 * glossary "vLLM": finished sequences return their blocks to the pool at once, continuous
 * batching entry; blocks shared across sequences, PagedAttention entry). It holds no
 * device memory and launches nothing; every call is O(number of ids named) and
 * serialized by an internal lock. Ids are 0 .. num_blocks - 1.
 *   create     a handle with every block free; free blocks are handed out most recently
 *              freed first, initially in ascending order. destroy releases the handle.
 *   alloc      n blocks with reference count 1 into ids_out[n], all or nothing
 *              (PA_ERR_EXHAUSTED, nothing changed, when fewer than n are free).
 *   share      one more reference to each listed block (an id may repeat); every id must
 *              be in use (PA_ERR_STATE, nothing changed).
 *   release    drop one reference per listed occurrence; blocks that reach zero return to
 *              the free list and are written to freed_out (capacity n, may be NULL) with
 *              their count in *num_freed (may be NULL). Fails with PA_ERR_STATE, nothing
 *              changed, if a block would go below zero. Freed FP4 blocks must be re-armed
 *              with pa_reset_blocks before their next first write.
 *   writable   copy on write for block `id` (in use): if it has one reference, *id_out = id
 *              and the call returns 0; otherwise a new block is allocated, id loses one
 *              reference, *id_out = the new block and the call returns 1: the caller then
 *              copies id -> *id_out with pa_copy_blocks. PA_ERR_EXHAUSTED if none is free.
 *   refcount   the block's reference count (0 when free), or PA_ERR_SHAPE out of range.
 *   num_free   the number of free blocks.
 * Out-of-range ids give PA_ERR_SHAPE, NULL pointers PA_ERR_NULL.
 */
typedef struct pa_block_allocator pa_block_allocator;
int pa_allocator_create(int32_t num_blocks, pa_block_allocator** out);
int pa_allocator_destroy(pa_block_allocator* a);
int pa_allocator_alloc(pa_block_allocator* a, int32_t n, int32_t* ids_out);
int pa_allocator_share(pa_block_allocator* a, const int32_t* ids, int32_t n);
int pa_allocator_release(pa_block_allocator* a, const int32_t* ids, int32_t n,
                         int32_t* freed_out, int32_t* num_freed);
int pa_allocator_writable(pa_block_allocator* a, int32_t id, int32_t* id_out);
int pa_allocator_refcount(pa_block_allocator* a, int32_t id);
int pa_allocator_num_free(pa_block_allocator* a);

/*
 * Paged decode for one query token per sequence.
 *   q             [num_seqs, num_q_heads, head_dim], dtype q_dtype
 *   block_tables  [num_seqs, max_blocks_per_seq] int32; entries past a sequence's last
 *                 block are never read
 *   context_lens  [num_seqs] int32, tokens to attend (including the token just written)
 *   sm_scale      softmax scale (1 / sqrt(head_dim) for the usual attention); a positive
 *                 finite number, else PA_ERR_SCALE (the kernels take each block's largest
 *                 logit as sm_scale times its largest dot product)
 *   partition_size 0: one pass per sequence; writes out [num_seqs, num_q_heads, head_dim]
 *                 fp32. Otherwise a positive multiple of 16: partition p of a sequence
 *                 covers tokens [p * ps, min((p + 1) * ps, L)); each partition with
 *                 p < ceil(L / ps) writes part_out[s, h, p, :] (its normalized output, fp32)
 *                 and part_lse[s, h, p] (natural-log log-sum-exp of its scaled logits);
 *                 part_out [num_seqs, num_q_heads, max_partitions, head_dim] and part_lse
 *                 [num_seqs, num_q_heads, max_partitions] with max_partitions =
 *                 ceil(max_blocks_per_seq * 16 / ps). Combine them with pa_merge.
 * The result is softmax attention over the dequantized cache, exactly as stored (the FP4
 * outlier terms are added to the compressed ones; dailyaiworld.com, "Technical
 * Breakdown", step 4). Asynchronous on `stream`.
 */
int pa_decode(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
              const pa_kv_pool* pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
              const int32_t* context_lens, float sm_scale, int32_t partition_size, float* out,
              float* part_out, float* part_lse, int32_t* dev_err, void* stream);

/*
 * One decode step in one launch: sequence s's new key and value rows, k_new[s] and v_new[s]
 * ([num_seqs, num_kv_heads, head_dim], q_dtype), are stored at its last position
 * L_s - 1 (slot block_tables[s][(L_s - 1) / 16] * 16 + (L_s - 1) % 16), byte for byte as
 * pa_cache_write stores them, and the sequence then attends over its L_s tokens exactly as
 * pa_decode. The cache write and the decode of a serving step (dailyaiworld.com, engine
 * diagram: new tokens go to the cache, then Flash-Decoding reads it) without a second
 * launch: the wave that reads position L_s - 1 writes it first. Every pool format; in an
 * FP4 pool a block the new row opens is calibrated on that row, as pa_cache_write does for
 * a call that puts one row into the block. The block must not be read by another sequence
 * of the batch (a shared block is copied first, pa_allocator_writable). A block id outside
 * the pool at that position is flagged and nothing is written there.
 * All other arguments, shapes and rules as pa_decode. Asynchronous on `stream`.
 */
int pa_append_decode(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                     const pa_kv_pool* pool, const void* k_new, const void* v_new,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, float sm_scale, int32_t partition_size,
                     float* out, float* part_out, float* part_lse, int32_t* dev_err,
                     void* stream);

/*
 * Paged attention for several query tokens per sequence, over the same pool: a chunk of a
 * long prompt processed after its keys and values were written (chunked prefill,
 * dailyaiworld.com, "vLLM 0.7 Ships Unified KV Cache Compression", engine diagram with
 * 512-token chunks; inferensys glossary "vLLM", chunked prefill entry), or the tokens a
 * draft model proposed, checked in one pass (inferensys glossary "vLLM", speculative
 * decoding entry).
 *   q             [num_queries, num_q_heads, head_dim], dtype q_dtype; sequence s owns
 *                 rows query_start[s] .. query_start[s + 1] - 1
 *   query_start   [num_seqs + 1] int32, device memory: row offsets into q and out
 *   max_query_len an upper bound on every sequence's query count n_s (sizes the grid)
 *   block_tables, context_lens, sm_scale as for pa_decode; context_lens[s] = L_s counts
 *                 the sequence's tokens including its n_s queries, whose keys and values
 *                 must already be in the pool
 *   out           [num_queries, num_q_heads, head_dim] fp32: query i of sequence s
 *                 (position L_s - n_s + i) attends causally to positions 0 .. L_s - n_s + i
 * The query group Hq / Hkv must divide 16. A sequence with n_s < 0, n_s > L_s,
 * n_s > max_query_len, rows outside [0, num_queries) or an invalid L_s is flagged
 * (PA_DEVERR_BAD_CONTEXT) and not read; its rows are zeroed when they lie inside
 * [0, num_queries) and n_s <= max_query_len. Asynchronous on `stream`.
 */
int pa_prefill(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
               int32_t num_queries, const int32_t* query_start, int32_t max_query_len,
               const pa_kv_pool* pool,
               const int32_t* block_tables, int32_t max_blocks_per_seq,
               const int32_t* context_lens, float sm_scale, float* out, int32_t* dev_err,
               void* stream);

/*
 * Launch geometry for tuning and tests. Every entry point picks its own geometry; the _ex
 * variants below take one of these (NULL, or a field 0, keeps the library's choice) and
 * are otherwise identical to the entry point they extend. The library reads no
 * environment variable and keeps no setting between calls.
 *   decode_waves       waves per decode workgroup: 1, 2, 4 or 8 (a workgroup covers one
 *                      partition of one (sequence, kv head); its waves take its blocks in
 *                      turn and merge their states in LDS)
 *   prefill_col_tiles  16-column MFMA tiles per pa_prefill wave: 2 or 3
 *   reserved           must be 0
 * Another value gives PA_ERR_SHAPE.
 */
typedef struct pa_launch_options {
  int32_t decode_waves;
  int32_t prefill_col_tiles;
  int32_t reserved[6];
} pa_launch_options;

int pa_decode_ex(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                 const pa_kv_pool* pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
                 const int32_t* context_lens, float sm_scale, int32_t partition_size, float* out,
                 float* part_out, float* part_lse, int32_t* dev_err,
                 const pa_launch_options* opts, void* stream);
int pa_append_decode_ex(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                        const pa_kv_pool* pool, const void* k_new, const void* v_new,
                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                        const int32_t* context_lens, float sm_scale, int32_t partition_size,
                        float* out, float* part_out, float* part_lse, int32_t* dev_err,
                        const pa_launch_options* opts, void* stream);
/*
 * pa_append_decode_ex with several new rows per sequence: k_new, v_new [num_seqs, new_tokens,
 * num_kv_heads, head_dim] (q_dtype); row i of sequence s is stored at its position
 * L_s - new_tokens + i, byte for byte as pa_cache_write stores it, by the wave that reads
 * that position, and the sequence then attends over its L_s tokens exactly as pa_decode.
 * For a step that appends a chunk of tokens to every sequence before attending (the
 * workload with a 512-token write per step: 8 rows for each of 64 sequences), or the
 * drafted tokens a verification step accepts (inferensys glossary "vLLM", speculative
 * decoding entry), in one launch. new_tokens = 1 is pa_append_decode_ex.
 *   new_tokens  1 .. max_blocks_per_seq * 16 (else PA_ERR_SHAPE); 16-bit and FP8 pools
 *               (a 4-bit block takes its outlier set from the rows of its first write,
 *               which a multi-row append would spread over several waves: an FP4 pool
 *               accepts new_tokens = 1 only, else PA_ERR_DTYPE)
 * A sequence with L_s < new_tokens is flagged (PA_DEVERR_BAD_CONTEXT), nothing of it is
 * written and it reads as an invalid context (zero output; split: every partition empty).
 * The new rows' blocks must not be read by another sequence of the batch.
 */
int pa_append_decode_n(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                       const pa_kv_pool* pool, const void* k_new, const void* v_new,
                       int32_t new_tokens, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens, float sm_scale,
                       int32_t partition_size, float* out, float* part_out, float* part_lse,
                       int32_t* dev_err, const pa_launch_options* opts, void* stream);
int pa_prefill_ex(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                  int32_t num_queries, const int32_t* query_start, int32_t max_query_len,
                  const pa_kv_pool* pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* context_lens, float sm_scale, float* out, int32_t* dev_err,
                  const pa_launch_options* opts, void* stream);

/*
 * Gather-only ceiling of the decode's access pattern, for measurement: the decode kernel
 * pa_decode_ex would launch for these arguments (same grid, waves, partitions, block
 * order) with its arithmetic compiled out. Every load the decode makes is kept - the
 * block-table entries, each attended (block, kv head) tile of K and V with the same
 * instructions and cache hints, the per-token scales, the 4-bit records and first outlier
 * slots, but not the queries - and the loaded words are XORed together so the loads stay. Its time is what the
 * decode's memory traffic alone costs on this GPU, the floor the decode's math must hide
 * under (the pages put the decode's limit on memory bandwidth: xonoai.com report on vLLM
 * v0.7.2, "Deconstructing the v0.7.2 Architecture").
 *   num_q_heads     the query group num_q_heads / num_kv_heads is checked as in pa_decode;
 *                   no query is read (0.1% of the decode's bytes at head_dim 128)
 *   sink            [1024] uint32, device memory: XORs of the loaded words (contents
 *                   meaningless; need not be zeroed)
 * Invalid block ids are skipped and flagged as in pa_decode. Asynchronous on `stream`.
 */
int pa_gather_probe(int32_t num_seqs, int32_t num_q_heads, const pa_kv_pool* pool,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t partition_size, uint32_t* sink,
                    int32_t* dev_err, const pa_launch_options* opts, void* stream);

/*
 * Log-sum-exp merge of pa_decode partitions: for each (s, h), over p < ceil(L_s / ps),
 * M = max lse_p, w_p = exp(lse_p - M), out = sum w_p o_p / sum w_p and, if lse_out is
 * not NULL, lse_out[s, h] = M + ln sum w_p. The pages name split-KV decoding
 * (Flash-Decoding, among the sources of dailyaiworld.com, "vLLM 0.7 Ships Unified KV
 * Cache Compression") but not the recombination; this is the standard exact identity for
 * softmax over a union of disjoint key sets, not a step the pages state. A partition whose
 * lse is not finite weighs 0 and its row is not read into the sum; a sequence with
 * L_s < 1 or L_s > max_partitions * partition_size (nothing its partitions can hold) gets
 * a zero output and lse -inf. Shapes as in pa_decode; out [num_seqs, num_q_heads,
 * head_dim] fp32, lse_out [num_seqs, num_q_heads] fp32. Asynchronous.
 */
int pa_merge(const float* part_out, const float* part_lse, const int32_t* context_lens,
             int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t max_partitions,
             int32_t partition_size, float* out, float* lse_out, void* stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. pa_decode with partition_size > 0
 * followed by pa_merge, with the partials (part_out, part_lse) in a library-owned static
 * device array of PA_STATIC_SCRATCH_BYTES instead of caller memory; the caller passes only
 * inputs and outputs (out [num_seqs, num_q_heads, head_dim] fp32, lse_out [num_seqs,
 * num_q_heads] fp32 or NULL, as pa_merge writes them). The call needs
 * num_seqs * num_q_heads * P * (head_dim + 1) * 4 bytes of it, P = ceil(max_blocks_per_seq
 * * 16 / partition_size); more gives PA_ERR_SCRATCH before anything is queued (32 MiB holds
 * 32 sequences of up to 122,880 tokens with 8 query heads at head_dim 128 and 512-token
 * partitions). It allocates nothing: each GPU holds its own copy of the array from the
 * library's first call on that device until the process ends, and the call looks up its
 * address on the current device. All calls on one GPU share that array, so calls that
 * overlap in time on one GPU (other streams, other host threads) race and must be
 * serialized by the caller; one call leaves its partials there until the next overwrites
 * them, and every row a call's merge reads is written by its decode first. Same
 * arguments, rules and results as pa_decode_ex (default launch) + pa_merge otherwise.
 * Asynchronous on `stream`.
 */
#define PA_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
int pa_decode_split_static(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                           const pa_kv_pool* pool, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           float sm_scale, int32_t partition_size, float* out, float* lse_out,
                           int32_t* dev_err, void* stream);

/* Host-only: a static, human-readable name for a pa_status value. */
const char* pa_status_string(int status);

/*
 * Copy the device error word to host memory (*host_out) and wait for it on `stream`.
 * dev_err is the device pointer passed to the other calls.
 */
int pa_read_device_error(const int32_t* dev_err, int32_t* host_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
