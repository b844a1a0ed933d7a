// Quantize kernels (the body is in tq_quantize_body.h) and their launcher.
#include "tq_quantize_body.h"

namespace tq {
namespace {

// Threads of a block.  The blocks that keep the fragments in LDS (128 KB at
// d=128) are one per CU; with 3-bit codes and bf16 input a wave fits in 168
// VGPRs, so 12 waves (3 per SIMD) share the fragments, else 8.
__host__ __device__ constexpr int quant_threads(bool use_lds, int w, bool bf16in) {
  return use_lds ? (w == 3 && bf16in ? 768 : 512) : 256;
}

template <int DPAD, bool BF16IN, bool USE_LDS, int NTL, int W, bool FULL, bool PLANES>
__global__ void __launch_bounds__(quant_threads(USE_LDS, W, BF16IN)) quantize_kernel(QArgs a) {
  constexpr int FR = (DPAD / 16) * (DPAD / 32);
  __shared__ Frag lds[USE_LDS ? 4 * FR * 64 : 1];
  quantize_body<DPAD, BF16IN, USE_LDS, NTL, W, FULL, quant_threads(USE_LDS, W, BF16IN), PLANES>(
      a, lds, blockIdx.x, gridDim.x);
}

// PLANES: MSE-only records (bit planes); W = 1 takes the stream form, which is
// the same bytes
template <int DPAD, bool BF16IN, bool USE_LDS, int NTL, bool FULL, bool PLANES>
int launch_w(const QArgs &a, int w, int blocks, hipStream_t s) {
  switch (w) {
#define TQ_W(W_, P_)                                                                                  \
    case W_:                                                                                          \
      quantize_kernel<DPAD, BF16IN, USE_LDS, NTL, W_, FULL, P_><<<blocks, quant_threads(USE_LDS, W_, BF16IN), 0, s>>>(a); \
      break;
    TQ_W(1, false) TQ_W(2, PLANES) TQ_W(3, PLANES) TQ_W(4, PLANES)
#undef TQ_W
    default: return TQ_ENOTSUP;
  }
  return hip_status();
}

template <int DPAD, bool USE_LDS, int NTL>
int launch_d(const QArgs &a, int w, bool bf16, int cus, hipStream_t s) {
  const int64_t per_block_tiles = quant_threads(USE_LDS, w, bf16) / 64;   // one tile per wave per pass
  const int64_t want = (a.ntiles + per_block_tiles - 1) / per_block_tiles;
  const int64_t cap = USE_LDS ? (int64_t)cus : (int64_t)cus * 4;
  const int blocks = (int)(want < cap ? (want > 0 ? want : 1) : cap);
  const bool full = a.d == DPAD && a.m == (a.prod ? DPAD : 0);
  if (full && a.prod)
    return bf16 ? launch_w<DPAD, true, USE_LDS, NTL, true, false>(a, w, blocks, s)
                : launch_w<DPAD, false, USE_LDS, NTL, true, false>(a, w, blocks, s);
  if (!a.prod)
    return bf16 ? launch_w<DPAD, true, USE_LDS, NTL, false, true>(a, w, blocks, s)
                : launch_w<DPAD, false, USE_LDS, NTL, false, true>(a, w, blocks, s);
  return bf16 ? launch_w<DPAD, true, USE_LDS, NTL, false, false>(a, w, blocks, s)
              : launch_w<DPAD, false, USE_LDS, NTL, false, false>(a, w, blocks, s);
}

}  // namespace

int launch_quantize(const tq_ctx *ctx, const void *x, int dtype, int64_t n, int64_t ldx,
                    int64_t ldr, uint8_t *codes, uint8_t *signs, float *norms, float *rnorms,
                    hipStream_t stream) {
  if (n == 0) return TQ_OK;
  if (ctx->frac) return launch_quantize_big(ctx, x, dtype, n, ldx, ldr, codes, signs, norms, rnorms, stream);
  QArgs a = make_qargs(ctx, x, n, ldx, ldr, codes, signs, norms, rnorms);
  const bool bf16 = dtype == TQ_BF16;
  const int w = ctx->hp.w;
  switch (ctx->dpad) {
    case 32:
      a.ntiles = (n + 31) / 32;
      return launch_d<32, true, 2>(a, w, bf16, ctx->cus, stream);
    case 64:
      a.ntiles = (n + 31) / 32;
      return launch_d<64, true, 2>(a, w, bf16, ctx->cus, stream);
    case 128:
      // few vectors (e.g. one decode token per KV head): 16-vector tiles, so
      // that twice as many waves share the work and each finishes sooner
      if (n <= 4096) {
        a.ntiles = (n + 15) / 16;
        return launch_d<128, true, 1>(a, w, bf16, ctx->cus, stream);
      }
      a.ntiles = (n + 31) / 32;
      return launch_d<128, true, 2>(a, w, bf16, ctx->cus, stream);
    case 256:
      a.ntiles = (n + 15) / 16;
      return launch_d<256, false, 1>(a, w, bf16, ctx->cus, stream);
    default:
      return launch_quantize_big(ctx, x, dtype, n, ldx, ldr, codes, signs, norms, rnorms, stream);
  }
}

}  // namespace tq
