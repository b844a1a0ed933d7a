// The small jobs of a decode step in one launch.
//
// Appending one token per KV group (a 16-vector tile per wave, a few
// microseconds of latency) and preparing the queries (one block per group,
// equally latency-bound) are independent; launched one after the other on a
// stream they cost their latencies in sequence.  This kernel gives each job
// its own blocks: blocks [0, kb) quantize the new keys, [kb, kb + vb) the new
// values, the rest prepare the queries (two 256-thread groups per block).
// The shared memory is a union of the quantizer's operand fragments and two
// prep work areas.
#include "tq_prep_body.h"
#include "tq_quantize_body.h"

namespace tq {
namespace {

constexpr int DEC_THREADS = 512;
constexpr int DEC_FR = (128 / 16) * (128 / 32);   // operand fragments per matrix at d = 128

template <bool BF16IN, int WK, int WV>
__global__ void __launch_bounds__(DEC_THREADS) decode_prep_kernel(QArgs qk, int kb, QArgs qv, int vb,
                                                                  PrepArgs pa, int groups) {
  __shared__ union {
    Frag lds[4 * DEC_FR * 64];
    PrepSmem<true> prep[2];
  } sm;
  const int b = blockIdx.x;
  if (b < kb) {
    quantize_body<128, BF16IN, true, 1, WK, true, DEC_THREADS>(qk, sm.lds, b, kb);
  } else if (WV > 0 && b < kb + vb) {
    // values: MSE-only records (bit planes)
    quantize_body<128, BF16IN, true, 1, (WV > 0 ? WV : 1), false, DEC_THREADS, true>(qv, sm.lds, b - kb, vb);
  } else {
    const int half = threadIdx.x >> 8;
    const int g = 2 * (b - kb - vb) + half;
    const bool live = g < groups;
    prep_body<128, true>(pa, sm.prep[half], live ? g : groups - 1, threadIdx.x & 255, live);
  }
}

template <bool BF16IN, int WK>
int launch_wv(int wv, const QArgs &qk, int kb, const QArgs &qv, int vb, const PrepArgs &pa, int groups,
              int blocks, hipStream_t s) {
  if (wv == 0)
    decode_prep_kernel<BF16IN, WK, 0><<<blocks, DEC_THREADS, 0, s>>>(qk, kb, qv, vb, pa, groups);
  else if (wv == WK + 1)      // values with as many bits per coordinate as the keys
    decode_prep_kernel<BF16IN, WK, WK + 1><<<blocks, DEC_THREADS, 0, s>>>(qk, kb, qv, vb, pa, groups);
  else
    return TQ_ENOTSUP;
  return hip_status();
}

}  // namespace

int launch_decode_prep(const tq_ctx *kc, const tq_ctx *vc, const float *q, int64_t G, int qpg,
                       const void *new_k, const void *new_v, int dtype, int64_t ldx, int64_t pos,
                       int64_t ldk, uint8_t *kcodes, uint8_t *ksigns, float *knorms, float *krnorms,
                       uint8_t *vcodes, float *vnorms, void *ws, hipStream_t stream) {
  // the fused launch covers d = 128 and up to 4096 groups (16-vector tiles);
  // everything else returns TQ_ENOTSUP and the caller launches the jobs apart
  if (kc->dpad != 128 || kc->hp.d != 128 || G > 4096) return TQ_ENOTSUP;
  if (vc && (vc->dpad != 128 || vc->hp.d != 128)) return TQ_ENOTSUP;
  const int wk = kc->hp.w, wv = vc ? vc->hp.w : 0;
  if (wk < 1 || wk > 3) return TQ_ENOTSUP;
  const int hg = (qpg + 3) / 4;
  const int64_t groups = G * hg;
  if (groups > 65535) return TQ_ENOTSUP;
  const int64_t tiles = (G + 15) / 16;
  const int kb = (int)((tiles + 7) / 8);                   // 8 waves per block, one tile each
  const int vb = vc ? kb : 0;
  const int pb = (int)((groups + 1) / 2);
  const QArgs qk = make_qargs(kc, new_k, G, ldx, ldk, kcodes + pos * kc->code_bytes,
                              ksigns + pos * kc->sign_bytes, knorms + pos, krnorms + pos);
  QArgs qv{};
  if (vc) qv = make_qargs(vc, new_v, G, ldx, ldk, vcodes + pos * vc->code_bytes, nullptr, vnorms + pos, nullptr);
  QArgs qk2 = qk, qv2 = qv;
  qk2.ntiles = tiles;
  qv2.ntiles = tiles;
  const PrepArgs pa = make_prep_args(kc, q, qpg, hg, G * qpg, reinterpret_cast<uint8_t *>(ws));
  const bool bf16 = dtype == TQ_BF16;
  const int blocks = kb + vb + pb;
  switch (wk) {
    case 1: return bf16 ? launch_wv<true, 1>(wv, qk2, kb, qv2, vb, pa, (int)groups, blocks, stream)
                        : launch_wv<false, 1>(wv, qk2, kb, qv2, vb, pa, (int)groups, blocks, stream);
    case 2: return bf16 ? launch_wv<true, 2>(wv, qk2, kb, qv2, vb, pa, (int)groups, blocks, stream)
                        : launch_wv<false, 2>(wv, qk2, kb, qv2, vb, pa, (int)groups, blocks, stream);
    default: return bf16 ? launch_wv<true, 3>(wv, qk2, kb, qv2, vb, pa, (int)groups, blocks, stream)
                         : launch_wv<false, 3>(wv, qk2, kb, qv2, vb, pa, (int)groups, blocks, stream);
  }
}

}  // namespace tq
