// pa_static.hip - split decode + merge with the partials in library-owned device memory,
// for callers that cannot allocate (pa_decode_split_static, include/pa.h).
//
// The split decode leaves one (o_p, lse_p) per partition that pa_merge then combines;
// pa_decode takes the buffers for them from the caller. Here they live in `scratch`, a
// file-scope device array of kScratchBytes that each GPU the library runs on holds until
// the process ends. Host code never passes the array's name to a kernel (on the host it
// only names a shadow variable): the first call on a device looks up the array's device
// address with hipGetSymbolAddress, with that device current, and keeps it per device.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/pa.h"

namespace {

constexpr size_t kScratchBytes = PA_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) static uint8_t scratch[kScratchBytes];

std::mutex g_lock;
void* g_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The device address of `scratch` on the current device (nullptr if it cannot be had).
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> hold(g_lock);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" int pa_decode_split_static(const void* q, int32_t q_dtype, int32_t num_seqs,
                                      int32_t num_q_heads, const pa_kv_pool* pool,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, float sm_scale,
                                      int32_t partition_size, float* out, float* lse_out,
                                      int32_t* dev_err, void* stream) {
  if (!pool) return PA_ERR_NULL;
  if (pool->head_dim != 64 && pool->head_dim != 128) return PA_ERR_SHAPE;
  if (num_seqs < 0 || num_q_heads < 1) return PA_ERR_SHAPE;
  if (partition_size <= 0 || partition_size % PA_BLOCK_SIZE != 0) return PA_ERR_PARTITION;
  if (max_blocks_per_seq < 1 || (int64_t)max_blocks_per_seq * PA_BLOCK_SIZE > INT32_MAX)
    return PA_ERR_CONTEXT;
  const int64_t P =
      ((int64_t)max_blocks_per_seq * PA_BLOCK_SIZE + partition_size - 1) / partition_size;
  const int64_t rows = (int64_t)num_seqs * num_q_heads * P;
  const int64_t out_bytes = rows * pool->head_dim * (int64_t)sizeof(float);
  const int64_t lse_bytes = rows * (int64_t)sizeof(float);
  if (out_bytes + lse_bytes > (int64_t)kScratchBytes) return PA_ERR_SCRATCH;
  if (num_seqs == 0) return PA_OK;
  // the merge's own checks, made before the decode is queued
  if (!out) return PA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(out) & 15) || (reinterpret_cast<uintptr_t>(lse_out) & 3))
    return PA_ERR_ALIGN;
  uint8_t* base = static_cast<uint8_t*>(scratch_ptr());
  if (!base) return PA_ERR_LAUNCH;
  // partials [S, Hq, P, D] at the start, lse [S, Hq, P] after them (a multiple of 256 bytes
  // in: D * 4 is 256 or 512). Every row the merge reads is written by the decode first
  // (an empty or unreadable partition too), so nothing needs clearing between calls.
  float* part_out = reinterpret_cast<float*>(base);
  float* part_lse = reinterpret_cast<float*>(base + out_bytes);
  int st = pa_decode_ex(q, q_dtype, num_seqs, num_q_heads, pool, block_tables,
                        max_blocks_per_seq, context_lens, sm_scale, partition_size, nullptr,
                        part_out, part_lse, dev_err, nullptr, stream);
  if (st != PA_OK) return st;
  return pa_merge(part_out, part_lse, context_lens, num_seqs, num_q_heads, pool->head_dim,
                  (int32_t)P, partition_size, out, lse_out, stream);
}
