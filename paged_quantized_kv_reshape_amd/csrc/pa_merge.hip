// pa_merge.hip - log-sum-exp merge of split-KV decode partitions (gfx950).
//
// Split-KV decode ("Flash-Decoding", dailyaiworld.com, "vLLM 0.7 Ships Unified KV Cache
// Compression", and its cited sources on parallel attention across compute units) leaves
// one normalized output o_p and one natural-log log-sum-exp lse_p per partition. The
// merge is exact: out = sum_p exp(lse_p - M) o_p / sum_p exp(lse_p - M), M = max_p lse_p,
// and the merged lse = M + ln sum_p exp(lse_p - M).
//
// One workgroup of W waves per (sequence, query head). Wave w folds partitions w, w + W,
// ... into (M_w, sum_w, acc_w) with its own maximum M_w (lane l owns channels D/64 l ..
// D/64 (l + 1) - 1, so each partition's row is one coalesced read); the W partial states
// are then combined through LDS. A long context (hundreds of partitions) is thus read by W waves
// in parallel instead of one, which keeps the merge bandwidth-bound.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

template <int D>
__global__ __launch_bounds__(1024) void k_merge(const float* __restrict__ po,
                                                const float* __restrict__ pl,
                                                const int32_t* __restrict__ cl, int32_t Hq,
                                                int32_t P, int32_t ps,
                                                float* __restrict__ out,
                                                float* __restrict__ lse_out) {
  constexpr int CPL = D / 64;  // channels per lane: lane l owns [CPL l, CPL (l + 1))
  typedef float vec_t __attribute__((ext_vector_type(CPL)));
  __shared__ float s_m[16], s_w[16];
  __shared__ vec_t s_acc[16][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int64_t sh = blockIdx.x;  // s * Hq + h
  const int s = (int)(sh / Hq);
  const int L = cl[s];
  const int np = L >= 1 ? min((L + ps - 1) / ps, P) : 0;
  vec_t* o = reinterpret_cast<vec_t*>(out + sh * D);
  if (np == 0) {
    if (wave == 0) {
      o[lane] = vec_t(0.0f);
      if (lse_out && lane == 0) lse_out[sh] = -INFINITY;
    }
    return;
  }
  const float* lse = pl + sh * P;
  float m = -INFINITY;
  for (int p = wave + W * lane; p < np; p += 64 * W) m = fmaxf(m, lse[p]);
  m = wave_max(m);
  vec_t acc = vec_t(0.0f);
  float wsum = 0.0f;
  const vec_t* base = reinterpret_cast<const vec_t*>(po + sh * (int64_t)P * D) + lane;
#pragma unroll 8
  for (int p = wave; p < np; p += W) {
    const float x = lse[p];
    const float w = x == -INFINITY ? 0.0f : __expf(x - m);
    wsum += w;
    acc += w * base[(int64_t)p * (D / CPL)];
  }
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
  // about 8 partitions per wave, 1..16 waves
  int waves = 1;
  while (waves < 16 && P > 8 * waves) waves *= 2;
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
