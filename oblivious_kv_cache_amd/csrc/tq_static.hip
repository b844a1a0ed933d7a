// tq_scores with its scratch memory inside the library: for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// tq_scores needs scratch memory for the prepared queries (the int8 operand
// fragments and per-head constants the query-prep kernel writes and the
// scores kernel reads).  Here that memory is one file-scope device array per
// GPU, `scratch`, of TQ_SCRATCH_BYTES.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in symbol): its device
// address is looked up once per device, with that device current, by
// hipGetSymbolAddress, and that address is what the kernels receive.
//
// Every call on one GPU shares that GPU's array, and the array keeps what the
// last call wrote: the prep kernel rewrites every byte the scores kernel
// reads, so nothing needs clearing, but calls that overlap in time on one GPU
// (on different streams, or from different threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "tq_internal.h"

static __device__ __align__(256) uint8_t scratch[TQ_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

}  // namespace

namespace tq {

void *scratch_attach(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[device]) return g_ptr[device];
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != device) return nullptr;
  void *p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
    (void)hipGetLastError();
    return nullptr;
  }
  g_ptr[device] = p;
  return p;
}

}  // namespace tq

extern "C" int tq_scores_static(const tq_ctx *ctx, const float *q, int64_t G, int qpg, int64_t T,
                                int64_t ldk, const uint8_t *codes, const uint8_t *signs,
                                const float *norms, const float *rnorms, float *logits,
                                hipStream_t stream) {
  int st = tq::check_scores_call(ctx, q, G, qpg, T, ldk, codes, signs, norms, rnorms, logits);
  if (st != TQ_OK || G == 0 || T == 0) return st;
  if (tq::scores_ws_bytes(ctx, G, qpg) > (size_t)TQ_SCRATCH_BYTES) return TQ_ESCRATCH;
  void *ws = tq::scratch_attach(ctx->device);     // set at tq_init; found again here
  if (!ws) return TQ_EHIP;
  return tq::launch_scores(ctx, q, G, qpg, T, ldk, codes, signs, norms, rnorms, logits, ws, stream);
}
