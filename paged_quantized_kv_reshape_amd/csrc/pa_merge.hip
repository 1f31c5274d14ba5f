// pa_merge.hip - log-sum-exp merge of split-KV decode partitions (gfx950).
//
// Split-KV decode ("Flash-Decoding", dailyaiworld.com, "vLLM 0.7 Ships Unified KV Cache
// Compression", and its cited sources on parallel attention across compute units) leaves
// one normalized output o_p and one natural-log log-sum-exp lse_p per partition. The
// merge is exact: out = sum_p exp(lse_p - M) o_p / sum_p exp(lse_p - M), M = max_p lse_p,
// and the merged lse = M + ln sum_p exp(lse_p - M).
//
// One wave per (sequence, query head); lane l owns channels {l, l + 64} (D = 128) or {l}
// (D = 64). The partitions' outputs are read once each, coalesced.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

template <int D>
__global__ __launch_bounds__(256) void k_merge(const float* __restrict__ po,
                                               const float* __restrict__ pl,
                                               const int32_t* __restrict__ cl, int32_t S,
                                               int32_t Hq, int32_t P, int32_t ps,
                                               float* __restrict__ out,
                                               float* __restrict__ lse_out) {
  constexpr int CPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t sh = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (sh >= (int64_t)S * Hq) return;
  const int s = (int)(sh / Hq);
  const int L = cl[s];
  const int np = L >= 1 ? min((L + ps - 1) / ps, P) : 0;
  float* o = out + sh * D;
  if (np == 0) {
#pragma unroll
    for (int k = 0; k < CPL; ++k) o[lane + 64 * k] = 0.0f;
    if (lse_out && lane == 0) lse_out[sh] = -INFINITY;
    return;
  }
  const float* lse = pl + sh * P;
  float M = -INFINITY;
  for (int p = lane; p < np; p += 64) M = fmaxf(M, lse[p]);
  M = wave_max(M);
  float acc[CPL], wsum = 0.0f;
#pragma unroll
  for (int k = 0; k < CPL; ++k) acc[k] = 0.0f;
  const float* base = po + sh * (int64_t)P * D;
#pragma unroll 4
  for (int p = 0; p < np; ++p) {
    const float x = lse[p];
    const float w = x == -INFINITY ? 0.0f : __expf(x - M);
    wsum += w;
#pragma unroll
    for (int k = 0; k < CPL; ++k) acc[k] = __builtin_fmaf(w, base[(int64_t)p * D + lane + 64 * k], acc[k]);
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
#pragma unroll
  for (int k = 0; k < CPL; ++k) o[lane + 64 * k] = acc[k] * inv;
  if (lse_out && lane == 0) lse_out[sh] = M + __logf(wsum);
}

int launch_merge(const float* part_out, const float* part_lse, const int32_t* context_lens,
                 int32_t S, int32_t Hq, int32_t D, int32_t P, int32_t ps, float* out,
                 float* lse_out, hipStream_t st) {
  const int64_t pairs = (int64_t)S * Hq;
  if (pairs == 0) return PA_OK;
  const dim3 grid((unsigned)((pairs + 3) / 4));
  if (D == 128)
    hipLaunchKernelGGL(k_merge<128>, grid, dim3(256), 0, st, part_out, part_lse, context_lens, S,
                       Hq, P, ps, out, lse_out);
  else
    hipLaunchKernelGGL(k_merge<64>, grid, dim3(256), 0, st, part_out, part_lse, context_lens, S,
                       Hq, P, ps, out, lse_out);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace pa
