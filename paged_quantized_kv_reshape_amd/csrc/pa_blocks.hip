// pa_blocks.hip - whole-block copies between paged pools on gfx950: the duplicate of a
// shared block that one of its sequences is about to extend (copy on write), and the swap
// of a preempted sequence's blocks to a pool in pinned host memory and back (inferensys
// glossary "vLLM": PagedAttention entry on blocks shared across sequences, preemption entry
// on swapping KV blocks to CPU RAM).
//
// One wave copies one pair: the block's bytes in every pool array (K, V and, for FP4, the
// two outlier-slot arrays), seen as one sequence of 16-byte vectors. Each lane loads up to
// kSlots vectors of that sequence before it stores any, so a wave keeps up to 8 KB in
// flight; with source and destination possibly in one pool the compiler could not move
// loads past stores by itself. Every array stores a block's bytes contiguously
// (block-major layout). Host-resident pools are read and written in place over the host
// link (pinned memory is mapped into the GPU's address space), so a swap is one pass with
// no staging buffer.
#include <hip/hip_runtime.h>

#include "../../include/pa.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kSlots = 8;

// a native 16-byte vector (HIP's uint4 is a struct, which keeps a register array of it
// from being promoted out of scratch memory)
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// NT: non-temporal loads and stores (each byte is read once and written once)
template <bool NT>
__global__ __launch_bounds__(64 * kWaves) void k_copy_blocks(CopyArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (pair >= a.num_pairs) return;
  const int2 pr = reinterpret_cast<const int2*>(a.pairs)[pair];
  const int32_t s = __builtin_amdgcn_readfirstlane(pr.x);
  const int32_t d = __builtin_amdgcn_readfirstlane(pr.y);
  if ((uint32_t)s >= (uint32_t)a.src_blocks || (uint32_t)d >= (uint32_t)a.dst_blocks) {
    if (lane == 0 && a.err) atomicOr(a.err, PA_DEVERR_BAD_BLOCK);
    return;
  }
  // the pair's vectors, array after array: [0, e0) in array 0, [e0, e1) in array 1, ...
  const uint32_t n0 = a.vecs_per_block[0], n1 = a.vecs_per_block[1];
  const uint32_t n2 = a.vecs_per_block[2], n3 = a.vecs_per_block[3];
  const uint32_t e0 = n0, e1 = e0 + n1, e2 = e1 + n2, total = e2 + n3;
  const v4u* s0 = reinterpret_cast<const v4u*>(a.src[0]) + (int64_t)s * n0;
  const v4u* s1 = reinterpret_cast<const v4u*>(a.src[1]) + (int64_t)s * n1;
  const v4u* s2 = reinterpret_cast<const v4u*>(a.src[2]) + (int64_t)s * n2;
  const v4u* s3 = reinterpret_cast<const v4u*>(a.src[3]) + (int64_t)s * n3;
  v4u* d0 = reinterpret_cast<v4u*>(a.dst[0]) + (int64_t)d * n0;
  v4u* d1 = reinterpret_cast<v4u*>(a.dst[1]) + (int64_t)d * n1;
  v4u* d2 = reinterpret_cast<v4u*>(a.dst[2]) + (int64_t)d * n2;
  v4u* d3 = reinterpret_cast<v4u*>(a.dst[3]) + (int64_t)d * n3;
  for (uint32_t base = 0; base < total; base += 64 * kSlots) {
    v4u r[kSlots];
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
      const uint32_t v = base + 64u * u + lane;
      // lanes past the end re-read the block's first vector (always in bounds), so the
      // loads need no branch; only the stores are masked
      const v4u* p = v < e0 || v >= total ? s0 : v < e1 ? s1 : v < e2 ? s2 : s3;
      const uint32_t o = v >= total ? 0u : v - (v < e0 ? 0u : v < e1 ? e0 : v < e2 ? e1 : e2);
      r[u] = NT ? __builtin_nontemporal_load(p + o) : p[o];
    }
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
      const uint32_t v = base + 64u * u + lane;
      v4u* p = v < e0 ? d0 : v < e1 ? d1 : v < e2 ? d2 : d3;
      const uint32_t o = v - (v < e0 ? 0u : v < e1 ? e0 : v < e2 ? e1 : e2);
      if (v < total) {
        if constexpr (NT)
          __builtin_nontemporal_store(r[u], p + o);
        else
          p[o] = r[u];
      }
    }
  }
}

}  // namespace

int launch_copy_blocks(const CopyArgs& a, hipStream_t st) {
  if (a.num_pairs == 0) return PA_OK;
  const int64_t gx = ((int64_t)a.num_pairs + kWaves - 1) / kWaves;
  if (a.streaming)
    hipLaunchKernelGGL(k_copy_blocks<true>, dim3((unsigned)gx), dim3(64 * kWaves), 0, st, a);
  else
    hipLaunchKernelGGL(k_copy_blocks<false>, dim3((unsigned)gx), dim3(64 * kWaves), 0, st, a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace pa
