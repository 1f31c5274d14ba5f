// pa_probe.hip - gather-only ceiling of the paged decode's memory traffic (gfx950).
//
// The decode is limited by memory bandwidth (xonoai.com field report on vLLM v0.7.2,
// "Deconstructing the v0.7.2 Architecture"), and its loads are scattered: every 16-token
// (block, kv head) run sits wherever the block table puts it. This kernel makes exactly the
// decode's launch (grid, waves per workgroup, partitions, the round-robin of a partition's
// blocks over the waves) and reads every byte of every attended K and V run through the
// block table with streaming 16-byte loads, but computes nothing: the words are XORed
// together so the loads cannot be removed. Its time is the floor the access pattern sets
// on this GPU, against which the decode's own time is judged.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// NV = 16-byte vectors per lane per run (a run of RB bytes is ceil(RB / 1024) wave loads);
// every block's K and V loads are issued before the XOR that consumes them, and two
// blocks are in flight per wave.
template <int NV>
__global__ __launch_bounds__(512) void k_gather_probe(DecodeArgs a, int32_t run_bytes,
                                                      uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int kvh = (int)(blockIdx.x % (unsigned)a.num_kv_heads);
  const int p = (int)(blockIdx.x / (unsigned)a.num_kv_heads);
  const int s = blockIdx.y;
  const int L = a.context_lens[s];
  const bool split = a.partition_size > 0;
  if (L < 1 || L > a.max_blocks * kBlock) {
    if (threadIdx.x == 0 && p == 0 && kvh == 0 && a.err) atomicOr(a.err, PA_DEVERR_BAD_CONTEXT);
    return;
  }
  const int start = split ? p * a.partition_size : 0;
  if (start >= L) return;
  const int end = split ? min(start + a.partition_size, L) : L;
  const int jb0 = start / kBlock;
  const int nblk = (end + kBlock - 1) / kBlock - jb0;
  const int my_n = wave < nblk ? (nblk - wave + W - 1) / W : 0;
  const int nvec = run_bytes / 16;  // vectors per run
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks + jb0 + wave;
  const uint8_t* kp = reinterpret_cast<const uint8_t*>(a.k);
  const uint8_t* vp = reinterpret_cast<const uint8_t*>(a.v);

  u32x4 acc = {0u, 0u, 0u, 0u};
  int err_bits = 0;
  int ids = 0;
  // lane j of a chunk holds the id of this wave's block 64 c + j
  for (int x = 0; x < my_n; x += 2) {
    if ((x & 63) == 0) {
      const int i = x + lane;
      ids = i < my_n ? bt[(int64_t)i * W] : 0;
    }
    u32x4 r[2][2][NV];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int xb = x + b;
      const int id = __builtin_amdgcn_readlane(ids, xb & 63);
      const bool live = xb < my_n;
      const bool ok = (unsigned)id < (unsigned)a.num_blocks;
      err_bits |= live && !ok ? PA_DEVERR_BAD_BLOCK : 0;
      const int64_t off = ((int64_t)(ok ? id : 0) * a.num_kv_heads + kvh) * run_bytes;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int v = j * 64 + lane;
        const bool take = live && ok && v < nvec;
        // lanes with nothing to read load the run's first vector again (in range, cached)
        const int64_t o = off + (take ? v : 0) * 16;
        r[b][0][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + o));
        r[b][1][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + o));
        if (!take) r[b][0][j] = r[b][1][j] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int j = 0; j < NV; ++j) acc ^= r[b][0][j] ^ r[b][1][j];
  }
  if (err_bits && lane == 0 && a.err) atomicOr(a.err, err_bits);
  uint32_t h = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) h ^= (uint32_t)__shfl_xor((int)h, o);
  if (lane == 0 && h != 0u) {
    const unsigned slot = (blockIdx.y * gridDim.x + blockIdx.x) * 8u + (unsigned)wave;
    atomicXor(sink + (slot & 1023u), h);
  }
}

}  // namespace

int launch_gather_probe(const DecodeArgs& a, int kv_dtype, int head_dim, int waves,
                        uint32_t* sink, hipStream_t st) {
  size_t b[4];
  const int rc = pa_pool_layout(kv_dtype, 1, 1, head_dim, b);
  if (rc != PA_OK) return rc;
  const int run_bytes = (int)b[0];  // bytes of one (block, kv head) run of K (V alike)
  const int nv = (run_bytes / 16 + 63) / 64;
  const int P = a.partition_size > 0 ? a.max_partitions : 1;
  const dim3 grid((unsigned)((int64_t)P * a.num_kv_heads), (unsigned)a.num_seqs, 1);
  const dim3 block(64 * waves);
  switch (nv) {
    case 1: hipLaunchKernelGGL(k_gather_probe<1>, grid, block, 0, st, a, run_bytes, sink); break;
    case 2: hipLaunchKernelGGL(k_gather_probe<2>, grid, block, 0, st, a, run_bytes, sink); break;
    case 3: hipLaunchKernelGGL(k_gather_probe<3>, grid, block, 0, st, a, run_bytes, sink); break;
    case 4: hipLaunchKernelGGL(k_gather_probe<4>, grid, block, 0, st, a, run_bytes, sink); break;
    default: return PA_ERR_SHAPE;
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace pa
