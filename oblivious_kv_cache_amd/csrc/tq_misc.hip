// Dequantization (reconstruction) kernel.
//
//   prod: x_hat = nu (Pi^T c[idx] + alpha gamma S^T (2 bits - 1))
//   mse:  x_hat = nu Pi^T c[idx]
//   fractional widths: as prod, with each half's centroids
//   polar: x_hat = nu Pi^T y_hat, y_hat the unit vector whose recursive polar
//          angles are the codes' centroid angles: coordinate i is the product,
//          over the levels l = 1..L of its path to the root, of the cosine
//          (child 0) or sine (child 1, bit l-1 of i) of the angle of node
//          i >> l (xujun.org note 189244, 第一步：PolarQuant)
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
  const float *pcs;   // polar mode: (cos, sin) of the angle centroids [L][2^w][2]; else null
  int nlev;           // polar mode: L = log2 d
  int frac, w2;       // fractional widths: second-half code bits and centroids
  float c2[16];
  int planes;         // MSE-only records: bit pl of code i at record bit pl d + i
};

// Record slot of the angle of node j at level l (polar layout: slots
// [q P, (q+1) P) of quarter q, P = d/4, hold its subtree level by level, then
// a spare slot: the top angle in quarter 0, the level L-1 angles in quarters
// 1 and 2).
__device__ __forceinline__ int polar_slot(int d, int L, int level, int j) {
  const int P = d >> 2;
  if (level == L) return P - 1;
  if (level == L - 1) return (j + 1) * P + P - 1;
  const int nq = P >> level, q = j / nq;
  return q * P + (P - (P >> (level - 1))) + (j - q * nq);
}

__global__ void __launch_bounds__(256) dequant_kernel(DqArgs a) {
  __shared__ float cv[TQ_MAX_D];
  __shared__ float sv[TQ_MAX_D];
  const int tid = threadIdx.x;
  for (int64_t v = blockIdx.x; v < a.n; v += gridDim.x) {
    const uint8_t *rec = a.codes + v * a.cb;
    auto code_at = [&](int slot) {
      const int bit = slot * a.w, byte = bit >> 3;
      uint32_t word = rec[byte];
      if (byte + 1 < a.cb) word |= (uint32_t)rec[byte + 1] << 8;
      return (word >> (bit & 7)) & ((1u << a.w) - 1u);
    };
    for (int j = tid; j < a.d; j += 256) {
      if (a.pcs) {
        float yv = 1.f;
        for (int level = 1; level <= a.nlev; ++level) {
          const uint32_t code = code_at(polar_slot(a.d, a.nlev, level, j >> level));
          yv *= a.pcs[(((level - 1) << a.w) + (int)code) * 2 + ((j >> (level - 1)) & 1)];
        }
        cv[j] = yv;
      } else if (a.frac) {
        // planar quarters: quarter g holds w_g bit planes of d/4 bits
        const int qd = a.d >> 2, g = j / qd, jq = j - g * qd;
        const int cw = g < 2 ? a.w : a.w2;
        const int base = 4 * (g < 2 ? g * a.w : 2 * a.w + (g - 2) * a.w2) * (qd >> 5);
        uint32_t code = 0;
        for (int pl = 0; pl < cw; ++pl) {
          const int bit = 8 * base + pl * qd + jq;
          code |= (uint32_t)((rec[bit >> 3] >> (bit & 7)) & 1) << pl;
        }
        cv[j] = g < 2 ? a.c[code] : a.c2[code];
      } else if (a.planes) {
        uint32_t code = 0;
        for (int pl = 0; pl < a.w; ++pl) {
          const int bit = pl * a.d + j;
          code |= (uint32_t)((rec[bit >> 3] >> (bit & 7)) & 1) << pl;
        }
        cv[j] = a.c[code];
      } else {
        cv[j] = a.c[code_at(j)];
      }
    }
    if (a.signs) {
      for (int k = tid; k < a.m; k += 256) {
        const uint8_t b = a.signs[v * a.sb + (k >> 3)];
        sv[k] = ((b >> (k & 7)) & 1) ? 1.f : -1.f;
      }
    }
    __syncthreads();
    for (int j = tid; j < a.d; j += 256) {
      float acc = 0.f;
      for (int i = 0; i < a.d; ++i) acc = fmaf(a.Pi[(int64_t)i * a.d + j], cv[i], acc);
      if (a.signs) {
        float acc2 = 0.f;
        for (int k = 0; k < a.m; ++k) acc2 = fmaf(a.S[(int64_t)k * a.d + j], sv[k], acc2);
        acc = fmaf(a.alpha * a.rnorms[v], acc2, acc);
      }
      a.out[v * a.d + j] = a.norms[v] * acc;
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
  for (int k = 0; k < 16; ++k) {
    a.c[k] = ctx->cf[k];
    a.c2[k] = ctx->cf2[k];
  }
  a.frac = ctx->frac;
  a.w2 = ctx->hp.w2;
  a.planes = ctx->hp.mode == TQ_MODE_MSE;
  a.pcs = ctx->hp.mode == TQ_MODE_POLAR ? ctx->polar_cs : nullptr;
  a.nlev = 0;
  while ((1 << a.nlev) < a.d) ++a.nlev;
  const int64_t blocks = n < 65536 ? n : 65536;
  dequant_kernel<<<(unsigned)blocks, 256, 0, stream>>>(a);
  return hip_status();
}

}  // namespace tq
