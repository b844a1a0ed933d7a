// Dequantization (reconstruction) kernel.
//
//   prod: x_hat = nu (Pi^T c[idx] + alpha gamma S^T (2 bits - 1))
//   mse:  x_hat = nu Pi^T c[idx]
// (suzuke blog "turboquant-compressing-ai-consciousness", 技術上怎麼做到的 /
// 第三步: the stage-1 approximation plus the residual correction).  Not on the
// timed path: a block per vector, decoded codes staged in LDS, then a
// coalesced pass over the rows of Pi and S.
#include "tq_internal.h"

namespace tq {
namespace {

struct DqArgs {
  const uint8_t *codes, *signs;
  const float *norms, *rnorms;
  float *out;
  const float *Pi, *S;
  int64_t n;
  int d, m, w, cb, sb;
  float alpha;
  float c[16];
};

__global__ void __launch_bounds__(256) dequant_kernel(DqArgs a) {
  __shared__ float cv[TQ_MAX_D];
  __shared__ float sv[TQ_MAX_D];
  const int tid = threadIdx.x;
  for (int64_t v = blockIdx.x; v < a.n; v += gridDim.x) {
    const uint8_t *rec = a.codes + v * a.cb;
    if (tid < a.d) {
      const int bit = tid * a.w, byte = bit >> 3;
      uint32_t word = rec[byte];
      if (byte + 1 < a.cb) word |= (uint32_t)rec[byte + 1] << 8;
      const uint32_t idx = (word >> (bit & 7)) & ((1u << a.w) - 1u);
      cv[tid] = a.c[idx];
    }
    if (a.signs && tid < a.m) {
      const uint8_t b = a.signs[v * a.sb + (tid >> 3)];
      sv[tid] = ((b >> (tid & 7)) & 1) ? 1.f : -1.f;
    }
    __syncthreads();
    if (tid < a.d) {
      float acc = 0.f;
      for (int i = 0; i < a.d; ++i) acc = fmaf(a.Pi[(int64_t)i * a.d + tid], cv[i], acc);
      if (a.signs) {
        float acc2 = 0.f;
        for (int k = 0; k < a.m; ++k) acc2 = fmaf(a.S[(int64_t)k * a.d + tid], sv[k], acc2);
        acc = fmaf(a.alpha * a.rnorms[v], acc2, acc);
      }
      a.out[v * a.d + tid] = a.norms[v] * acc;
    }
    __syncthreads();
  }
}

}  // namespace

int launch_dequant(const tq_ctx *ctx, const uint8_t *codes, const uint8_t *signs,
                   const float *norms, const float *rnorms, int64_t n, float *out,
                   hipStream_t stream) {
  DqArgs a{};
  a.codes = codes;
  a.signs = signs;
  a.norms = norms;
  a.rnorms = rnorms;
  a.out = out;
  a.Pi = ctx->Pi32;
  a.S = ctx->S32;
  a.n = n;
  a.d = ctx->hp.d;
  a.m = ctx->hp.m;
  a.w = ctx->hp.w;
  a.cb = ctx->code_bytes;
  a.sb = ctx->sign_bytes;
  a.alpha = ctx->alpha;
  for (int k = 0; k < 16; ++k) a.c[k] = ctx->cf[k];
  const int64_t blocks = n < 65536 ? n : 65536;
  dequant_kernel<<<(unsigned)blocks, 256, 0, stream>>>(a);
  return hip_status();
}

}  // namespace tq
