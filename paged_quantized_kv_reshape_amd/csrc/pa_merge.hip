// pa_merge.hip - log-sum-exp merge of split-KV decode partitions (gfx950).
//
// Split-KV decode ("Flash-Decoding", dailyaiworld.com, "vLLM 0.7 Ships Unified KV Cache
// Compression", and its cited sources on parallel attention across compute units) leaves
// one normalized output o_p and one natural-log log-sum-exp lse_p per partition. The
// merge is exact: out = sum_p exp(lse_p - M) o_p / sum_p exp(lse_p - M), M = max_p lse_p,
// and the merged lse = M + ln sum_p exp(lse_p - M).
//
// One workgroup of W waves per (sequence, query head). The partitions go to the waves in
// batches of 16: wave w takes partitions 16 w .. 16 w + 15, then 16 (w + W) .. and so on.
// A batch costs one trip to memory: lane j loads lse of the batch's partition j and the
// wave loads the batch's 16 rows (lane l holds channels D/64 l .. D/64 (l + 1) - 1 of each,
// so a row is one coalesced read, a batch 16 consecutive rows), all before any of them is
// used. Slots past the last partition re-read the last row (in range, and cached) with
// weight 0. A wave rescales its running state (M_w, weight sum, acc_w) when a batch raises
// its maximum; the W states are then combined through LDS. The merge is bound by the
// latency of that one trip, not by the bytes: a context of a few hundred partitions is read
// by every wave of the workgroup at once.
#include <algorithm>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kMergeBatch = 16;  // partitions per wave and trip
constexpr int kMergeMaxWaves = 16;

template <int D>
__global__ __launch_bounds__(64 * kMergeMaxWaves) void k_merge(
    const float* __restrict__ po, const float* __restrict__ pl, const int32_t* __restrict__ cl,
    int32_t Hq, int32_t P, int32_t ps, float* __restrict__ out, float* __restrict__ lse_out) {
  constexpr int CPL = D / 64;  // channels per lane: lane l owns [CPL l, CPL (l + 1))
  constexpr int B = kMergeBatch;
  typedef float vec_t __attribute__((ext_vector_type(CPL)));
  __shared__ float s_m[kMergeMaxWaves], s_w[kMergeMaxWaves];
  __shared__ vec_t s_acc[kMergeMaxWaves][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int64_t sh = blockIdx.x;  // s * Hq + h
  const int s = (int)(sh / Hq);
  const int L = cl[s];
  // a context the P partitions cannot hold (or none at all) has nothing valid to merge
  const int np = L >= 1 && (int64_t)L <= (int64_t)P * ps ? (L + ps - 1) / ps : 0;
  vec_t* o = reinterpret_cast<vec_t*>(out + sh * D);
  if (np == 0) {
    if (wave == 0) {
      o[lane] = vec_t(0.0f);
      if (lse_out && lane == 0) lse_out[sh] = -INFINITY;
    }
    return;
  }
  const float* lse = pl + sh * P;
  const vec_t* rows = reinterpret_cast<const vec_t*>(po + sh * (int64_t)P * D) + lane;
  float m = -INFINITY;  // this wave's running maximum (wave-uniform)
  float wl = 0.0f;      // this lane's share of the weight sum
  vec_t acc = vec_t(0.0f);
  for (int b0 = wave * B; b0 < np; b0 += W * B) {
    // a non-finite lse (nothing written there that a decode would write) weighs 0
    float x = lane < B && b0 + lane < np ? lse[b0 + lane] : -INFINITY;
    x = __builtin_isfinite(x) ? x : -INFINITY;
    vec_t r[B];
#pragma unroll
    for (int j = 0; j < B; ++j) r[j] = rows[(int64_t)min(b0 + j, np - 1) * (D / CPL)];
    const float mn = fmaxf(m, wave_max(x));
    if (mn == -INFINITY) continue;  // no finite lse yet: the state is still all zero
    if (mn > m) {
      const float f = m == -INFINITY ? 0.0f : __expf(m - mn);
      acc *= f;
      wl *= f;
      m = mn;
    }
    const float wx = x == -INFINITY ? 0.0f : __expf(x - m);
    wl += wx;
#pragma unroll
    for (int j = 0; j < B; ++j) {
      // a row of weight 0 is skipped, not multiplied: its values may be anything (NaN)
      const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wx), j));
      if (wj != 0.0f) acc += wj * r[j];
    }
  }
  const float wsum = wave_sum(wl);
  if (W == 1) {
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    o[lane] = acc * inv;
    if (lse_out && lane == 0) lse_out[sh] = m + __logf(wsum);
    return;
  }
  if (lane == 0) {
    s_m[wave] = m;  // -inf for a wave that saw no partition
    s_w[wave] = wsum;
  }
  s_acc[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  float M = -INFINITY;
  for (int w = 0; w < W; ++w) M = fmaxf(M, s_m[w]);
  float tot = 0.0f;
  vec_t o_acc = vec_t(0.0f);
  for (int w = 0; w < W; ++w) {
    const float f = s_m[w] == -INFINITY ? 0.0f : __expf(s_m[w] - M);
    tot += f * s_w[w];
    o_acc += f * s_acc[w][lane];
  }
  const float inv = tot > 0.0f ? 1.0f / tot : 0.0f;
  o[lane] = o_acc * inv;
  if (lse_out && lane == 0) lse_out[sh] = M + __logf(tot);
}

int launch_merge(const float* part_out, const float* part_lse, const int32_t* context_lens,
                 int32_t S, int32_t Hq, int32_t D, int32_t P, int32_t ps, float* out,
                 float* lse_out, hipStream_t st) {
  const int64_t pairs = (int64_t)S * Hq;
  if (pairs == 0) return PA_OK;
  // one batch of partitions per wave where that takes at most 16 waves
  const int waves = (int)std::min<int64_t>(kMergeMaxWaves,
                                           std::max<int64_t>(1, ((int64_t)P + kMergeBatch - 1) /
                                                                    kMergeBatch));
  const dim3 grid((unsigned)pairs);
  if (D == 128)
    hipLaunchKernelGGL(k_merge<128>, grid, dim3(64 * waves), 0, st, part_out, part_lse,
                       context_lens, Hq, P, ps, out, lse_out);
  else
    hipLaunchKernelGGL(k_merge<64>, grid, dim3(64 * waves), 0, st, part_out, part_lse,
                       context_lens, Hq, P, ps, out, lse_out);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace pa
