// Host-only stand-ins for the HIP runtime and the kernel launchers, so that
// the library's host code (parameter construction, context set-up, argument
// validation) can be built with the address and undefined-behaviour
// sanitizers and run without a GPU.  Device memory is host memory here and
// every launcher does nothing; only the host logic around them is exercised.
#include <hip/hip_runtime_api.h>

#include <cstdlib>
#include <cstring>

#include "../../oblivious_kv_cache_amd/csrc/tq_internal.h"

hipError_t hipGetDevice(int *d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int *v, hipDeviceAttribute_t, int) {
  *v = 256;
  return hipSuccess;
}
hipError_t hipMalloc(void **p, size_t n) {
  *p = std::malloc(n ? n : 1);
  return *p ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipFree(void *p) {
  std::free(p);
  return hipSuccess;
}
hipError_t hipMemcpy(void *dst, const void *src, size_t n, hipMemcpyKind) {
  std::memcpy(dst, src, n);
  return hipSuccess;
}
hipError_t hipGetLastError() { return hipSuccess; }

namespace tq {

int launch_quantize(const tq_ctx *, const void *, int, int64_t, int64_t, int64_t, uint8_t *, uint8_t *,
                    float *, float *, hipStream_t) {
  return TQ_OK;
}
int launch_polar_quantize(const tq_ctx *, const void *, int, int64_t, int64_t, int64_t, uint8_t *, float *,
                          hipStream_t) {
  return TQ_OK;
}
size_t scores_ws_bytes(const tq_ctx *, int64_t G, int qpg) { return (size_t)(G * ((qpg + 3) / 4)) * 1024; }
int launch_scores(const tq_ctx *, const float *, int64_t, int, int64_t, int64_t, const uint8_t *,
                  const uint8_t *, const float *, const float *, float *, void *, hipStream_t) {
  return TQ_OK;
}
int launch_prep_queries(const tq_ctx *, const float *, int64_t, int, void *, hipStream_t) { return TQ_OK; }
int launch_scores_prepared(const tq_ctx *, const void *, int64_t, int, int64_t, int64_t, const uint8_t *,
                           const uint8_t *, const float *, const float *, float *, hipStream_t, hipEvent_t,
                           hipEvent_t) {
  return TQ_OK;
}
int launch_softmax(const float *, int64_t, int64_t, float, float *, hipStream_t) { return TQ_OK; }
int launch_dequant(const tq_ctx *, const uint8_t *, const uint8_t *, const float *, const float *, int64_t,
                   float *, hipStream_t) {
  return TQ_OK;
}
size_t attend_ws_bytes(const tq_ctx *, int64_t G, int qpg, int64_t T) {
  return (size_t)(G * qpg) * (size_t)(T + 1) * 8;
}
int check_attend(const tq_ctx *, const tq_ctx *, int64_t, int, int64_t, int64_t, bool) { return TQ_OK; }
int launch_attend(const tq_ctx *, const tq_ctx *, const float *, int64_t, int, int64_t, int64_t,
                  const uint8_t *, const uint8_t *, const float *, const float *, const uint8_t *,
                  const float *, float, float *, float *, float *, void *, hipStream_t, bool) {
  return TQ_OK;
}
int launch_decode_prep(const tq_ctx *, const tq_ctx *, const float *, int64_t, int, const void *, const void *,
                       int, int64_t, int64_t, int64_t, uint8_t *, uint8_t *, float *, float *, uint8_t *, float *,
                       void *, hipStream_t) {
  return TQ_ENOTSUP;
}
size_t topk_ws_bytes(const tq_ctx *, int64_t nq, int64_t n, int k) { return (size_t)(nq * k + n) * 8; }
int launch_topk(const tq_ctx *, const float *, int64_t, int64_t, const uint8_t *, const uint8_t *,
                const float *, const float *, int, int64_t *, float *, void *, hipStream_t) {
  return TQ_OK;
}
void *scratch_attach(int) {
  static unsigned char dummy[256];
  return dummy;
}

}  // namespace tq
