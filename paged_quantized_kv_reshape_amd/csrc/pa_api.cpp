// pa_api.cpp - the C ABI of libpa (declared in include/pa.h): host-side argument checks,
// launch geometry, status strings. Every check runs before any HIP call, so a rejected
// call has no effect on the device.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pa.h"
#include "pa_launch.h"

namespace {

constexpr int64_t kMaxGridYZ = 65535;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Format, shape, block arrays and their alignment; not the per-head scales.
int check_pool_arrays(const pa_kv_pool* p) {
  if (!p) return PA_ERR_NULL;
  if (p->dtype < PA_KV_F16 || p->dtype > PA_KV_FP8_E5M2_TOKEN) return PA_ERR_DTYPE;
  if (p->block_size != PA_BLOCK_SIZE) return PA_ERR_BLOCK_SIZE;
  if (p->num_blocks < 1 || p->num_kv_heads < 1 || p->num_kv_heads > kMaxGridYZ)
    return PA_ERR_SHAPE;
  if (p->head_dim != 64 && p->head_dim != 128) return PA_ERR_SHAPE;
  if ((int64_t)p->num_blocks * PA_BLOCK_SIZE > INT64_C(0x3FFFFFFFFFFFFFFF)) return PA_ERR_SHAPE;
  if (!p->k || !p->v) return PA_ERR_NULL;
  if (!aligned(p->k, 16) || !aligned(p->v, 16)) return PA_ERR_ALIGN;
  if (p->dtype == PA_KV_FP4_E2M1_OUTL) {
    if (!p->k_out_val || !p->v_out_val) return PA_ERR_NULL;
    if (!aligned(p->k_out_val, 8) || !aligned(p->v_out_val, 8)) return PA_ERR_ALIGN;
  }
  return PA_OK;
}

int check_pool(const pa_kv_pool* p) {
  const int st = check_pool_arrays(p);
  if (st != PA_OK) return st;
  if (p->dtype == PA_KV_FP8_E4M3 || p->dtype == PA_KV_FP8_E5M2) {
    if (!p->k_scale || !p->v_scale) return PA_ERR_NULL;
    if (!aligned(p->k_scale, 4) || !aligned(p->v_scale, 4)) return PA_ERR_ALIGN;
  }
  return PA_OK;
}

// True when the current GPU can dereference p at address p: its own device memory, or
// pinned host memory mapped at the same address. Pageable host memory, which the runtime
// does not know, is refused (a kernel touching it would fault).
bool gpu_accessible(const void* p) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();  // leave no error behind for the next launch check
    return false;
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (at.type == hipMemoryTypeDevice) return at.device == dev;
  if (at.type == hipMemoryTypeHost || at.type == hipMemoryTypeManaged)
    return at.devicePointer == p;
  return false;
}

bool act_ok(int32_t act) { return act == PA_ACT_F16 || act == PA_ACT_BF16; }

// A 16-bit pool stores the activation dtype itself.
bool act_matches_pool(int32_t act, int32_t kv) {
  if (kv == PA_KV_F16) return act == PA_ACT_F16;
  if (kv == PA_KV_BF16) return act == PA_ACT_BF16;
  return true;
}

// Compute units of the current device (256 on MI355X if the query fails).
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    return 256;
  return n;
}

// Launch options: NULL or zero fields keep the library's choice; anything else must be a
// value the kernels are built for.
int check_options(const pa_launch_options* o) {
  if (!o) return PA_OK;
  const int w = o->decode_waves;
  if (w != 0 && w != 1 && w != 2 && w != 4 && w != 8) return PA_ERR_SHAPE;
  if (o->prefill_col_tiles != 0 && o->prefill_col_tiles != 2 && o->prefill_col_tiles != 3)
    return PA_ERR_SHAPE;
  for (int i = 0; i < 6; ++i)
    if (o->reserved[i] != 0) return PA_ERR_SHAPE;
  return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: a size is out of range or inconsistent";
    case PA_ERR_DTYPE: return "PA_ERR_DTYPE: unknown or unsupported dtype combination";
    case PA_ERR_BLOCK_SIZE: return "PA_ERR_BLOCK_SIZE: block_size must be 16";
    case PA_ERR_CONTEXT: return "PA_ERR_CONTEXT: max_blocks_per_seq out of range";
    case PA_ERR_PARTITION: return "PA_ERR_PARTITION: partition_size must be 0 or a positive multiple of 16";
    case PA_ERR_LAUNCH: return "PA_ERR_LAUNCH: the HIP runtime refused a launch";
    case PA_ERR_ALIGN: return "PA_ERR_ALIGN: a pointer is not suitably aligned";
    case PA_ERR_MEMORY: return "PA_ERR_MEMORY: a pointer is not memory this GPU can access";
    case PA_ERR_EXHAUSTED: return "PA_ERR_EXHAUSTED: not enough free blocks";
    case PA_ERR_STATE: return "PA_ERR_STATE: the block is not in use";
    case PA_ERR_SCRATCH:
      return "PA_ERR_SCRATCH: the call needs more device scratch than the library holds";
    case PA_ERR_SCALE: return "PA_ERR_SCALE: sm_scale must be a positive finite number";
    default: return "unknown pa_status";
  }
}

int pa_outlier_capacity(int32_t head_dim) {
  const int c = pa::outlier_capacity(head_dim);
  return c < 0 ? PA_ERR_SHAPE : c;
}

int pa_pool_layout(int32_t dtype, int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                   size_t bytes_out[4]) {
  if (!bytes_out) return PA_ERR_NULL;
  if (dtype < PA_KV_F16 || dtype > PA_KV_FP8_E5M2_TOKEN) return PA_ERR_DTYPE;
  if (num_blocks < 1 || num_kv_heads < 1 || (head_dim != 64 && head_dim != 128))
    return PA_ERR_SHAPE;
  for (int i = 0; i < 4; ++i) bytes_out[i] = 0;
  const size_t bh = (size_t)num_blocks * num_kv_heads;
  const size_t rows = bh * PA_BLOCK_SIZE;
  switch (dtype) {
    case PA_KV_F16:
    case PA_KV_BF16: bytes_out[0] = bytes_out[1] = rows * head_dim * 2; break;
    case PA_KV_FP8_E4M3:
    case PA_KV_FP8_E5M2: bytes_out[0] = bytes_out[1] = rows * head_dim; break;
    case PA_KV_FP8_E4M3_TOKEN:
    case PA_KV_FP8_E5M2_TOKEN:
      bytes_out[0] = bh * (size_t)PA_FP8T_TILE_BYTES(head_dim);
      bytes_out[1] = bh * (size_t)PA_FP8T_VTILE_BYTES(head_dim);
      break;
    default:
      bytes_out[0] = bytes_out[1] = bh * (size_t)PA_FP4_TILE_BYTES(head_dim);
      bytes_out[2] = bytes_out[3] = bh * (size_t)(pa::outlier_capacity(head_dim) - 1) *
                                    PA_BLOCK_SIZE * sizeof(uint16_t);
  }
  return PA_OK;
}

int pa_cache_write(const pa_kv_pool* pool, const void* k_new, const void* v_new, int32_t act,
                   int32_t num_tokens, const int64_t* slot_mapping, int32_t* dev_err,
                   void* stream) {
  int st = check_pool(pool);
  if (st != PA_OK) return st;
  if (!act_ok(act) || !act_matches_pool(act, pool->dtype)) return PA_ERR_DTYPE;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping) return PA_ERR_NULL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(slot_mapping, 8) ||
      !aligned(dev_err, 4))
    return PA_ERR_ALIGN;
  return pa::launch_write(*pool, k_new, v_new, act == PA_ACT_BF16, num_tokens, slot_mapping,
                          dev_err, (hipStream_t)stream);
}

int pa_fp8_head_scales(const void* x, int32_t act, int32_t kv_dtype, int64_t num_rows,
                       int32_t num_kv_heads, int32_t head_dim, float* scale_out, void* stream) {
  if (!act_ok(act)) return PA_ERR_DTYPE;
  if (kv_dtype != PA_KV_FP8_E4M3 && kv_dtype != PA_KV_FP8_E5M2) return PA_ERR_DTYPE;
  if (num_rows < 0 || num_kv_heads < 1 || num_kv_heads > 256 ||
      (head_dim != 64 && head_dim != 128))
    return PA_ERR_SHAPE;
  if (!scale_out || (num_rows > 0 && !x)) return PA_ERR_NULL;
  if (!aligned(x, 16) || !aligned(scale_out, 4)) return PA_ERR_ALIGN;
  return pa::launch_fp8_scales(x, act == PA_ACT_BF16, kv_dtype == PA_KV_FP8_E5M2, num_rows,
                               num_kv_heads, head_dim, scale_out, (hipStream_t)stream);
}

int pa_fp4_sequence_outliers(const void* k_rows, const void* v_rows, int32_t act,
                             int64_t num_rows, int32_t num_kv_heads, int32_t head_dim,
                             const int32_t* row_start, int32_t num_seqs, uint8_t* seq_records,
                             int32_t* dev_err, void* stream) {
  if (!act_ok(act)) return PA_ERR_DTYPE;
  if ((head_dim != 64 && head_dim != 128) || num_rows < 0 || num_seqs < 0 || num_kv_heads < 1 ||
      num_kv_heads > kMaxGridYZ)
    return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!row_start || !seq_records || (num_rows > 0 && (!k_rows || !v_rows))) return PA_ERR_NULL;
  if (!aligned(k_rows, 16) || !aligned(v_rows, 16) || !aligned(row_start, 4) ||
      !aligned(seq_records, 16) || !aligned(dev_err, 4))
    return PA_ERR_ALIGN;
  return pa::launch_fp4_seq_outliers(k_rows, v_rows, act == PA_ACT_BF16, num_rows, num_kv_heads,
                                     head_dim, row_start, num_seqs, seq_records, dev_err,
                                     (hipStream_t)stream);
}

int pa_cache_write_seq_outliers(const pa_kv_pool* pool, const void* k_new, const void* v_new,
                                int32_t act, int32_t num_tokens, const int64_t* slot_mapping,
                                const int32_t* token_seq, const uint8_t* seq_records,
                                int32_t num_seqs, int32_t* dev_err, void* stream) {
  int st = check_pool(pool);
  if (st != PA_OK) return st;
  if (pool->dtype != PA_KV_FP4_E2M1_OUTL || !act_ok(act)) return PA_ERR_DTYPE;
  if (num_tokens < 0 || num_seqs < 0) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping || !token_seq || !seq_records) return PA_ERR_NULL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(slot_mapping, 8) ||
      !aligned(token_seq, 4) || !aligned(seq_records, 16) || !aligned(dev_err, 4))
    return PA_ERR_ALIGN;
  return pa::launch_write(*pool, k_new, v_new, act == PA_ACT_BF16, num_tokens, slot_mapping,
                          dev_err, (hipStream_t)stream, token_seq, seq_records, num_seqs);
}

int pa_reset_blocks(const pa_kv_pool* pool, const int32_t* block_ids, int32_t n, void* stream) {
  int st = check_pool(pool);
  if (st != PA_OK) return st;
  if (n < 0) return PA_ERR_SHAPE;
  if (pool->dtype != PA_KV_FP4_E2M1_OUTL || n == 0) return PA_OK;
  if (!block_ids) return PA_ERR_NULL;
  if (!aligned(block_ids, 4)) return PA_ERR_ALIGN;
  return pa::launch_reset(*pool, block_ids, n, (hipStream_t)stream);
}

int pa_copy_blocks(const pa_kv_pool* src, const pa_kv_pool* dst, const int32_t* pairs,
                   int32_t num_pairs, int32_t* dev_err, void* stream) {
  int st = check_pool_arrays(src);
  if (st != PA_OK) return st;
  if ((st = check_pool_arrays(dst)) != PA_OK) return st;
  if (src->dtype != dst->dtype) return PA_ERR_DTYPE;
  if (src->num_kv_heads != dst->num_kv_heads || src->head_dim != dst->head_dim)
    return PA_ERR_SHAPE;
  if (num_pairs < 0) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!pairs) return PA_ERR_NULL;
  if (!aligned(pairs, 8) || !aligned(dev_err, 4)) return PA_ERR_ALIGN;
  size_t sb[4], db[4];
  if ((st = pa_pool_layout(src->dtype, src->num_blocks, src->num_kv_heads, src->head_dim, sb)) !=
      PA_OK)
    return st;
  if ((st = pa_pool_layout(dst->dtype, dst->num_blocks, dst->num_kv_heads, dst->head_dim, db)) !=
      PA_OK)
    return st;
  pa::CopyArgs a{};
  const void* sp[4] = {src->k, src->v, src->k_out_val, src->v_out_val};
  void* dp[4] = {dst->k, dst->v, dst->k_out_val, dst->v_out_val};
  for (int j = 0; j < 4; ++j) {
    if (sb[j] == 0) continue;
    const size_t per_block = sb[j] / (size_t)src->num_blocks;
    if (per_block % 16 != 0 || per_block / 16 > UINT32_MAX) return PA_ERR_SHAPE;
    if (!aligned(sp[j], 16) || !aligned(dp[j], 16)) return PA_ERR_ALIGN;
    a.src[a.num_arrays] = sp[j];
    a.dst[a.num_arrays] = dp[j];
    a.vecs_per_block[a.num_arrays] = (uint32_t)(per_block / 16);
    ++a.num_arrays;
  }
  // A swap names memory on the host: check that the GPU can reach every pointer. Within
  // one pool (copy on write) the arrays are the decode's own device memory and, as for
  // the other entry points, are not looked up.
  bool same = true;
  for (int j = 0; j < a.num_arrays; ++j) same = same && a.src[j] == a.dst[j];
  if (!same) {
    for (int j = 0; j < a.num_arrays; ++j)
      if (!gpu_accessible(a.src[j]) || !gpu_accessible(a.dst[j])) return PA_ERR_MEMORY;
    if (!gpu_accessible(pairs) || (dev_err && !gpu_accessible(dev_err))) return PA_ERR_MEMORY;
  }
  a.pairs = pairs;
  a.num_pairs = num_pairs;
  a.src_blocks = src->num_blocks;
  a.dst_blocks = dst->num_blocks;
  a.err = dev_err;
  // within one pool both sides are device memory read and written once: streaming loads
  // and stores (measured: 4.82 -> 5.06 TB/s for 65536 FP8 blocks); a swap touches pinned
  // host memory, where the hint cost 1% (54.5 -> 54.1 GB/s), so it keeps the plain form
  a.streaming = same;
  return pa::launch_copy_blocks(a, (hipStream_t)stream);
}

}  // extern "C"

namespace {

// Checks shared by the decode entry points and the gather probe: the pool, the GQA group,
// the table and partition sizes. Fills the launch arguments common to them.
int decode_geometry(int32_t num_seqs, int32_t num_q_heads, const pa_kv_pool* pool,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t partition_size,
                    const pa_launch_options* opts, pa::DecodeArgs& a) {
  int st = check_pool(pool);
  if (st != PA_OK) return st;
  if ((st = check_options(opts)) != PA_OK) return st;
  if (num_seqs < 0 || num_seqs > kMaxGridYZ || num_q_heads < 1) return PA_ERR_SHAPE;
  if (num_q_heads % pool->num_kv_heads != 0) return PA_ERR_SHAPE;
  const int group = num_q_heads / pool->num_kv_heads;
  if (group > 16) return PA_ERR_SHAPE;
  if (max_blocks_per_seq < 1 || (int64_t)max_blocks_per_seq * PA_BLOCK_SIZE > INT32_MAX)
    return PA_ERR_CONTEXT;
  if (partition_size < 0 || partition_size % PA_BLOCK_SIZE != 0) return PA_ERR_PARTITION;
  const int64_t cap_tokens = (int64_t)max_blocks_per_seq * PA_BLOCK_SIZE;
  const int max_part =
      partition_size > 0 ? (int)((cap_tokens + partition_size - 1) / partition_size) : 1;
  // the launch grid's x dimension counts (partition, kv head) pairs
  if ((int64_t)max_part * pool->num_kv_heads > INT32_MAX) return PA_ERR_SHAPE;
  if (num_seqs > 0 && (!block_tables || !context_lens)) return PA_ERR_NULL;
  if (!aligned(block_tables, 4) || !aligned(context_lens, 4)) return PA_ERR_ALIGN;
  a.k = pool->k;
  a.v = pool->v;
  a.k_out_val = pool->k_out_val;
  a.v_out_val = pool->v_out_val;
  a.k_scale = pool->k_scale;
  a.v_scale = pool->v_scale;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.group = group;
  a.num_blocks = pool->num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.partition_size = partition_size;
  a.max_partitions = max_part;
  a.cap = pa::outlier_capacity(pool->head_dim);
  return PA_OK;
}

// The softmax scale: positive (a block's largest logit is then the scale times its largest
// dot product, which the multi-token kernel relies on) and finite; NaN fails both tests.
bool scale_ok(float s) { return s > 0.0f && s <= 3.4028234663852886e38f; }

// K + V bytes of one (block, kv head) tile of a pool format.
size_t tile_pair_bytes(int32_t dtype, int32_t head_dim) {
  switch (dtype) {
    case PA_KV_F16:
    case PA_KV_BF16: return (size_t)2 * PA_BLOCK_SIZE * head_dim * 2;
    case PA_KV_FP8_E4M3:
    case PA_KV_FP8_E5M2: return (size_t)2 * PA_BLOCK_SIZE * head_dim;
    case PA_KV_FP4_E2M1_OUTL: return (size_t)2 * PA_FP4_TILE_BYTES(head_dim);
    default: return (size_t)PA_FP8T_TILE_BYTES(head_dim) + PA_FP8T_VTILE_BYTES(head_dim);
  }
}

// Waves per decode workgroup. The decode streams K/V tiles from HBM. Measured on MI355X,
// two rules, the larger count wins (a power of two up to 8, doubled only while the
// partition has at least two blocks per wave):
//  * occupancy: with one kv head the gather of random 16-token tiles runs fastest with
//    about 8 waves per compute unit in the grid (more waves only open more DRAM rows at
//    once); with several kv heads the workgroups of one block's heads run side by side and
//    read neighbouring tiles, and about 8 waves per CU per kv head (up to 8 heads) keeps
//    those reads together. FP4 pools start from 2 waves: a 4-bit tile is half an FP8 one,
//    so a one-wave workgroup keeps too little in flight, and the FP4 kernel's wave merge
//    reuses its own LDS, so two waves cost no occupancy (FP4, 32 x 64k-120k tokens: 107 us
//    vs 113 us with one).
//  * work per wave: about 48 KiB of K/V per wave of a partition. A workgroup's waves
//    finish together and the last workgroups of a launch run with the GPU part idle, so
//    a shorter wave shortens that tail, down to where its fixed costs (the query, the
//    block ids, the wave merge) start to count. Sweeps of partition size and waves
//    found the best at 6 bf16 (64 x 1k-8k tokens, 8 kv heads, 768-token partitions, 8
//    waves), 12 FP8 (the same shapes, 768, 4 waves) and 16 FP4 tiles (32 x 64k-120k tokens,
//    512, 2 waves) per wave: 48, 48 and 37 KiB.
int decode_waves(const pa::DecodeArgs& a, int32_t dtype, int32_t head_dim,
                 const pa_launch_options* opts) {
  if (opts && opts->decode_waves) return opts->decode_waves;
  const int64_t span = a.partition_size > 0 ? a.partition_size
                                            : (int64_t)a.max_blocks * PA_BLOCK_SIZE;
  const int64_t blocks = (span + PA_BLOCK_SIZE - 1) / PA_BLOCK_SIZE;
  const int64_t wgs = (int64_t)a.num_seqs * a.num_kv_heads * a.max_partitions;
  const int64_t heads = a.num_kv_heads < 8 ? a.num_kv_heads : 8;
  const int64_t target_waves = 8 * heads * (int64_t)device_cus();
  const int64_t bytes = blocks * (int64_t)tile_pair_bytes(dtype, head_dim);
  int waves = dtype == PA_KV_FP4_E2M1_OUTL && blocks >= 4 ? 2 : 1;
  while (waves < 8 && blocks >= 2 * waves &&
         (wgs * waves < target_waves || bytes > (int64_t)waves * (48 << 10)))
    waves *= 2;
  return waves;
}

// pa_decode and pa_append_decode[_n]: k_new / v_new NULL for the former; n_new new rows
// per sequence for the latter
int decode_call(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                const pa_kv_pool* pool, const void* k_new, const void* v_new, int32_t n_new,
                const int32_t* block_tables, int32_t max_blocks_per_seq,
                const int32_t* context_lens, float sm_scale, int32_t partition_size, float* out,
                float* part_out, float* part_lse, int32_t* dev_err,
                const pa_launch_options* opts, void* stream) {
  pa::DecodeArgs a{};
  int st = decode_geometry(num_seqs, num_q_heads, pool, block_tables, max_blocks_per_seq,
                           context_lens, partition_size, opts, a);
  if (st != PA_OK) return st;
  if (!act_ok(q_dtype) || !act_matches_pool(q_dtype, pool->dtype)) return PA_ERR_DTYPE;
  if (!scale_ok(sm_scale)) return PA_ERR_SCALE;
  if (num_seqs == 0) return PA_OK;
  if (!q) return PA_ERR_NULL;
  if (partition_size == 0) {
    if (!out) return PA_ERR_NULL;
    if (!aligned(out, 16)) return PA_ERR_ALIGN;
  } else {
    if (!part_out || !part_lse) return PA_ERR_NULL;
    if (!aligned(part_out, 16) || !aligned(part_lse, 4)) return PA_ERR_ALIGN;
  }
  if (!aligned(q, 16) || !aligned(dev_err, 4) || !aligned(k_new, 16) || !aligned(v_new, 16))
    return PA_ERR_ALIGN;
  if (k_new) {
    if (n_new < 1 || (int64_t)n_new > (int64_t)max_blocks_per_seq * PA_BLOCK_SIZE)
      return PA_ERR_SHAPE;
    // a 4-bit block takes its outlier set from the rows of its first write, which several
    // new rows per sequence would spread over several waves
    if (n_new > 1 && pool->dtype == PA_KV_FP4_E2M1_OUTL) return PA_ERR_DTYPE;
  }
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_tokens = k_new ? n_new : 0;
  a.out = out;
  a.part_out = part_out;
  a.part_lse = part_lse;
  a.err = dev_err;
  a.sm_scale_log2 = sm_scale * 1.4426950408889634f;
  return pa::launch_decode(a, pool->dtype, q_dtype == PA_ACT_BF16, pool->head_dim,
                           decode_waves(a, pool->dtype, pool->head_dim, opts), (hipStream_t)stream);
}

int prefill_call(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                 int32_t num_queries, const int32_t* query_start, int32_t max_query_len,
                 const pa_kv_pool* pool, const int32_t* block_tables,
                 int32_t max_blocks_per_seq, const int32_t* context_lens, float sm_scale,
                 float* out, int32_t* dev_err, const pa_launch_options* opts, void* stream) {
  int st = check_pool(pool);
  if (st != PA_OK) return st;
  if ((st = check_options(opts)) != PA_OK) return st;
  if (!act_ok(q_dtype) || !act_matches_pool(q_dtype, pool->dtype)) return PA_ERR_DTYPE;
  if (!scale_ok(sm_scale)) return PA_ERR_SCALE;
  if (num_seqs < 0 || num_seqs > kMaxGridYZ || num_q_heads < 1) return PA_ERR_SHAPE;
  if (num_q_heads % pool->num_kv_heads != 0) return PA_ERR_SHAPE;
  const int group = num_q_heads / pool->num_kv_heads;
  if (16 % group != 0) return PA_ERR_SHAPE;  // a wave's 16 columns hold whole queries
  if (max_query_len < 0 || num_queries < 0) return PA_ERR_SHAPE;
  if (max_blocks_per_seq < 1 || (int64_t)max_blocks_per_seq * PA_BLOCK_SIZE > INT32_MAX)
    return PA_ERR_CONTEXT;
  if (num_seqs == 0 || max_query_len == 0 || num_queries == 0) return PA_OK;
  if (!q || !query_start || !block_tables || !context_lens || !out) return PA_ERR_NULL;
  // the grid's x dimension counts (query tile, kv head) pairs
  if ((int64_t)max_query_len * pool->num_kv_heads > INT32_MAX) return PA_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(query_start, 4) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(dev_err, 4))
    return PA_ERR_ALIGN;

  pa::DecodeArgs a{};
  a.q = q;
  a.k = pool->k;
  a.v = pool->v;
  a.k_out_val = pool->k_out_val;
  a.v_out_val = pool->v_out_val;
  a.k_scale = pool->k_scale;
  a.v_scale = pool->v_scale;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.out = out;
  a.err = dev_err;
  a.query_start = query_start;
  a.max_query_len = max_query_len;
  a.num_queries = num_queries;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.group = group;
  a.num_blocks = pool->num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.partition_size = 0;
  a.max_partitions = 1;
  a.cap = pa::outlier_capacity(pool->head_dim);
  a.sm_scale_log2 = sm_scale * 1.4426950408889634f;
  return pa::launch_prefill(a, pool->dtype, q_dtype == PA_ACT_BF16, pool->head_dim,
                            opts ? opts->prefill_col_tiles : 0, (hipStream_t)stream);
}

}  // namespace

extern "C" {

int pa_decode(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
              const pa_kv_pool* pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
              const int32_t* context_lens, float sm_scale, int32_t partition_size, float* out,
              float* part_out, float* part_lse, int32_t* dev_err, void* stream) {
  return decode_call(q, q_dtype, num_seqs, num_q_heads, pool, nullptr, nullptr, 0, block_tables,
                     max_blocks_per_seq, context_lens, sm_scale, partition_size, out, part_out,
                     part_lse, dev_err, nullptr, stream);
}

int pa_decode_ex(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                 const pa_kv_pool* pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
                 const int32_t* context_lens, float sm_scale, int32_t partition_size, float* out,
                 float* part_out, float* part_lse, int32_t* dev_err,
                 const pa_launch_options* opts, void* stream) {
  return decode_call(q, q_dtype, num_seqs, num_q_heads, pool, nullptr, nullptr, 0, block_tables,
                     max_blocks_per_seq, context_lens, sm_scale, partition_size, out, part_out,
                     part_lse, dev_err, opts, stream);
}

int pa_append_decode(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                     const pa_kv_pool* pool, const void* k_new, const void* v_new,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, float sm_scale, int32_t partition_size,
                     float* out, float* part_out, float* part_lse, int32_t* dev_err,
                     void* stream) {
  return pa_append_decode_ex(q, q_dtype, num_seqs, num_q_heads, pool, k_new, v_new,
                             block_tables, max_blocks_per_seq, context_lens, sm_scale,
                             partition_size, out, part_out, part_lse, dev_err, nullptr, stream);
}

int pa_append_decode_ex(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                        const pa_kv_pool* pool, const void* k_new, const void* v_new,
                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                        const int32_t* context_lens, float sm_scale, int32_t partition_size,
                        float* out, float* part_out, float* part_lse, int32_t* dev_err,
                        const pa_launch_options* opts, void* stream) {
  return pa_append_decode_n(q, q_dtype, num_seqs, num_q_heads, pool, k_new, v_new, 1,
                            block_tables, max_blocks_per_seq, context_lens, sm_scale,
                            partition_size, out, part_out, part_lse, dev_err, opts, stream);
}

int pa_append_decode_n(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                       const pa_kv_pool* pool, const void* k_new, const void* v_new,
                       int32_t new_tokens, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens, float sm_scale,
                       int32_t partition_size, float* out, float* part_out, float* part_lse,
                       int32_t* dev_err, const pa_launch_options* opts, void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new)) return PA_ERR_NULL;
  if (new_tokens < 1) return PA_ERR_SHAPE;
  return decode_call(q, q_dtype, num_seqs, num_q_heads, pool, k_new, v_new, new_tokens,
                     block_tables, max_blocks_per_seq, context_lens, sm_scale, partition_size,
                     out, part_out, part_lse, dev_err, opts, stream);
}

int pa_prefill(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
               int32_t num_queries, const int32_t* query_start, int32_t max_query_len,
               const pa_kv_pool* pool,
               const int32_t* block_tables, int32_t max_blocks_per_seq,
               const int32_t* context_lens, float sm_scale, float* out, int32_t* dev_err,
               void* stream) {
  return prefill_call(q, q_dtype, num_seqs, num_q_heads, num_queries, query_start,
                      max_query_len, pool, block_tables, max_blocks_per_seq, context_lens,
                      sm_scale, out, dev_err, nullptr, stream);
}

int pa_prefill_ex(const void* q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads,
                  int32_t num_queries, const int32_t* query_start, int32_t max_query_len,
                  const pa_kv_pool* pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* context_lens, float sm_scale, float* out, int32_t* dev_err,
                  const pa_launch_options* opts, void* stream) {
  return prefill_call(q, q_dtype, num_seqs, num_q_heads, num_queries, query_start,
                      max_query_len, pool, block_tables, max_blocks_per_seq, context_lens,
                      sm_scale, out, dev_err, opts, stream);
}

int pa_gather_probe(int32_t num_seqs, int32_t num_q_heads, const pa_kv_pool* pool,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t partition_size, uint32_t* sink,
                    int32_t* dev_err, const pa_launch_options* opts, void* stream) {
  pa::DecodeArgs a{};
  int st = decode_geometry(num_seqs, num_q_heads, pool, block_tables, max_blocks_per_seq,
                           context_lens, partition_size, opts, a);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return PA_OK;
  if (!sink) return PA_ERR_NULL;
  if (!aligned(sink, 4) || !aligned(dev_err, 4)) return PA_ERR_ALIGN;
  a.err = dev_err;
  return pa::launch_gather_probe(a, pool->dtype, pool->head_dim,
                                 decode_waves(a, pool->dtype, pool->head_dim, opts), sink, (hipStream_t)stream);
}

int pa_merge(const float* part_out, const float* part_lse, const int32_t* context_lens,
             int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t max_partitions,
             int32_t partition_size, float* out, float* lse_out, void* stream) {
  if (num_seqs < 0 || num_q_heads < 1 || (head_dim != 64 && head_dim != 128) ||
      max_partitions < 1)
    return PA_ERR_SHAPE;
  if (partition_size <= 0 || partition_size % PA_BLOCK_SIZE != 0) return PA_ERR_PARTITION;
  if (num_seqs == 0) return PA_OK;
  if (!part_out || !part_lse || !context_lens || !out) return PA_ERR_NULL;
  if (!aligned(part_out, 16) || !aligned(part_lse, 4) || !aligned(context_lens, 4) ||
      !aligned(out, 16) || !aligned(lse_out, 4))
    return PA_ERR_ALIGN;
  return pa::launch_merge(part_out, part_lse, context_lens, num_seqs, num_q_heads, head_dim,
                          max_partitions, partition_size, out, lse_out, (hipStream_t)stream);
}

int pa_read_device_error(const int32_t* dev_err, int32_t* host_out, void* stream) {
  if (!dev_err || !host_out) return PA_ERR_NULL;
  hipStream_t st = (hipStream_t)stream;
  if (hipMemcpyAsync(host_out, dev_err, sizeof(int32_t), hipMemcpyDeviceToHost, st) != hipSuccess)
    return PA_ERR_LAUNCH;
  return hipStreamSynchronize(st) == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // extern "C"
