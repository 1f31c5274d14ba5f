// Host-only stand-ins for libpa's kernel launchers, for the sanitizer build of the C ABI
// (pa_api.cpp and pa_alloc.cpp under AddressSanitizer / UndefinedBehaviorSanitizer on the
// CPU). Each returns PA_ERR_LAUNCH: in this build a call that passes every host check
// reaches a launcher and reports that nothing ran. Test infrastructure only.
#include "../../paged_quantized_kv_reshape_amd/csrc/pa_launch.h"

namespace pa {

int launch_write(const pa_kv_pool&, const void*, const void*, bool, int32_t, const int64_t*,
                 int32_t*, hipStream_t, const int32_t*, const uint8_t*, int32_t) {
  return PA_ERR_LAUNCH;
}
int launch_fp4_seq_outliers(const void*, const void*, bool, int64_t, int32_t, int32_t,
                            const int32_t*, int32_t, uint8_t*, int32_t*, hipStream_t) {
  return PA_ERR_LAUNCH;
}
int launch_fp8_scales(const void*, bool, bool, int64_t, int32_t, int32_t, float*, hipStream_t) {
  return PA_ERR_LAUNCH;
}
int launch_reset(const pa_kv_pool&, const int32_t*, int32_t, hipStream_t) { return PA_ERR_LAUNCH; }
int launch_decode(const DecodeArgs&, int, bool, int, int, hipStream_t) { return PA_ERR_LAUNCH; }
int launch_gather_probe(const DecodeArgs&, int, int, int, uint32_t*, hipStream_t) {
  return PA_ERR_LAUNCH;
}
int launch_prefill(const DecodeArgs&, int, bool, int, int, hipStream_t) { return PA_ERR_LAUNCH; }
int launch_copy_blocks(const CopyArgs&, hipStream_t) { return PA_ERR_LAUNCH; }
int launch_merge(const float*, const float*, const int32_t*, int32_t, int32_t, int32_t, int32_t,
                 int32_t, float*, float*, hipStream_t) {
  return PA_ERR_LAUNCH;
}

}  // namespace pa

// The static-scratch decode lives in a HIP source (its device array); here it only reports
// that nothing ran, so the binding finds every symbol it binds.
extern "C" int pa_decode_split_static(const void*, int32_t, int32_t, int32_t, const pa_kv_pool*,
                                      const int32_t*, int32_t, const int32_t*, float, int32_t,
                                      float*, float*, int32_t*, void*) {
  return PA_ERR_LAUNCH;
}
