// C ABI entry points: argument validation, context construction and upload.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <new>

#include "tq_internal.h"

namespace {

using tq::Frag;

uint16_t bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)(u >> 16);   // inf / nan
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
float bf16_to_f(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// hi/lo bf16 split of a float64 value: hi = bf16(x), lo = bf16(x - hi).
void split_bf16(double x, uint16_t &hi, uint16_t &lo) {
  hi = bf16_rne((float)x);
  lo = bf16_rne((float)(x - (double)bf16_to_f(hi)));
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// contexts whose records carry a QJL sketch (the estimator's inputs)
bool scoring_mode(const tq_ctx *ctx) {
  return ctx->hp.mode == TQ_MODE_PROD || ctx->hp.mode == TQ_MODE_FRAC;
}

int current_device_matches(const tq_ctx *ctx) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return TQ_EHIP;
  return dev == ctx->device ? TQ_OK : TQ_EINVAL;
}

// Operand fragments of the quantize kernel (see tq_quantize.hip).  For output
// tile u, k-block k, lane l (row r = l % 16, k-group g = l / 16), element e:
//   GEMM 1: A = Pi[sigma(u, r)][32 k + 8 g + e]
//   GEMM 2: A = S'[sigma(u, r)][g * P + 8 k + e]      (S' = S Pi^T, P = dpad/4)
// with the row permutation sigma(u, r) = (r / 4) * P + 4 u + (r % 4), which
// hands lane group g the coordinates [g P, (g+1) P).
//
// For the kernel that stages vectors in LDS (d > 256, and the fractional
// widths) there is no permutation: row = 16 u + r and column 32 k + 8 g + e
// for both GEMMs.
void build_frags(const tq::HostParams &hp, int dpad, const double *M, int rows, int cols,
                 bool gemm2, bool plain, Frag *hi, Frag *lo) {
  const int NT = dpad / 16, NK = dpad / 32, P = dpad / 4;
  for (int u = 0; u < NT; ++u)
    for (int k = 0; k < NK; ++k)
      for (int l = 0; l < 64; ++l) {
        const int r = l % 16, g = l / 16;
        const int row = plain ? 16 * u + r : (r / 4) * P + 4 * u + (r % 4);
        uint16_t h8[8], l8[8];
        for (int e = 0; e < 8; ++e) {
          const int c = (gemm2 && !plain) ? g * P + 8 * k + e : 32 * k + 8 * g + e;
          double v = 0.0;
          if (row < rows && c < cols) v = M[(size_t)row * cols + c];
          split_bf16(v, h8[e], l8[e]);
        }
        Frag fh, fl;
        for (int i = 0; i < 4; ++i) {
          fh.v[i] = (uint32_t)h8[2 * i] | ((uint32_t)h8[2 * i + 1] << 16);
          fl.v[i] = (uint32_t)l8[2 * i] | ((uint32_t)l8[2 * i + 1] << 16);
        }
        const size_t idx = ((size_t)u * NK + k) * 64 + l;
        hi[idx] = fh;
        lo[idx] = fl;
      }
  (void)hp;
}

int make_ctx(int d, int bits, uint64_t seed, int mode, tq_ctx **out) {
  if (!out) return TQ_EINVAL;
  tq_ctx *ctx = new (std::nothrow) tq_ctx;
  if (!ctx) return TQ_ENOMEM;
  int st = tq::build_host_params(d, bits, seed, mode, ctx->hp);
  if (st != TQ_OK) {
    delete ctx;
    return st;
  }
  const tq::HostParams &hp = ctx->hp;
  const int m = hp.m, w = hp.w, L = hp.levels;
  const bool frac = mode == TQ_MODE_FRAC;
  ctx->frac = frac ? 1 : 0;
  ctx->dpad = d <= 32 ? 32 : d <= 64 ? 64 : d <= 128 ? 128 : d <= 256 ? 256 : (d + 31) / 32 * 32;
  // fractional mode: planar quarters, no padding (d in {128, 256})
  ctx->code_bytes = frac ? d * (w + hp.w2) / 16 : ((d * w + 7) / 8 + 15) / 16 * 16;
  ctx->sign_bytes = m ? ((m + 7) / 8 + 15) / 16 * 16 : 0;
  ctx->cw16 = frac ? w * d / 128 : ctx->code_bytes / 16;
  ctx->alpha = m ? (float)(std::sqrt(M_PI / 2.0) / m) : 0.f;
  // centroids (all, and the positive half), positive thresholds, and the odd
  // multilinear coefficients of the antisymmetric codebook in the sign
  // variables s_p = 2 bit_p - 1 (p = 0..w-1) and, for w = 3, s0 s1 s2
  auto codebook = [](const std::vector<double> &c, const std::vector<double> &t, int cw, float *cf,
                     float *cpos, float *tpos, float *basis) {
    const int n = 1 << cw;
    for (int k = 0; k < n; ++k) cf[k] = (float)c[k];
    for (int j = 0; j < n / 2; ++j) cpos[j] = (float)c[n / 2 + j];
    for (int j = 0; j + 1 < n / 2; ++j) tpos[j] = (float)t[n / 2 + j];
    for (int p = 0; p < 4; ++p) {
      double acc = 0.0;
      for (int idx = 0; idx < n; ++idx) {
        double s;
        if (p < cw && p < 3) {
          s = ((idx >> p) & 1) ? 1.0 : -1.0;
        } else if (p == 3 && cw == 3) {
          s = 1.0;
          for (int b = 0; b < 3; ++b) s *= ((idx >> b) & 1) ? 1.0 : -1.0;
        } else {
          s = 0.0;
        }
        acc += c[idx] * s;
      }
      basis[p] = (float)(acc / n);
    }
  };
  if (mode != TQ_MODE_POLAR) codebook(hp.c, hp.t, w, ctx->cf, ctx->cpos, ctx->tpos, ctx->basis);
  if (frac) codebook(hp.c2, hp.t2, hp.w2, ctx->cf2, ctx->cpos2, ctx->tpos2, ctx->basis2);
  // the same expansion with every odd monomial of up to 4 code bits: the w
  // single bits, then the products of three bits (w = 3: {012}; w = 4:
  // {012, 013, 023, 123}); used by the value sum of the attention kernel
  {
    static const int tri[4][3] = {{0, 1, 2}, {0, 1, 3}, {0, 2, 3}, {1, 2, 3}};
    const int ntri = w == 3 ? 1 : w == 4 ? 4 : 0;
    for (int p = 0; p < w + ntri; ++p) {
      double acc = 0.0;
      for (int idx = 0; idx < L; ++idx) {
        double s = 1.0;
        if (p < w) {
          s = ((idx >> p) & 1) ? 1.0 : -1.0;
        } else {
          for (int b = 0; b < 3; ++b) s *= ((idx >> tri[p - w][b]) & 1) ? 1.0 : -1.0;
        }
        acc += hp.c[idx] * s;
      }
      ctx->vbasis[p] = (float)(acc / L);
    }
  }

  if (hipGetDevice(&ctx->device) != hipSuccess) {
    delete ctx;
    return TQ_EHIP;
  }
  {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, ctx->device) == hipSuccess && v > 0)
      ctx->cus = v;
  }
  const int dpad = ctx->dpad;
  const size_t nfr = (size_t)(dpad / 16) * (dpad / 32) * 64;
  const size_t bytes_f32 = sizeof(float) * ((size_t)2 * d * d + (size_t)2 * m * d);
  const size_t bytes_fr = sizeof(Frag) * nfr * (m ? 4 : 2);
  // polar mode: per level, the angle thresholds [L][levels-1] and the
  // (cos, sin) of the angle centroids [L][levels][2], float32
  const bool polar = mode == TQ_MODE_POLAR;
  const int nlev = polar ? (int)std::lround(std::log2((double)d)) : 0;
  const size_t n_thr = polar ? (size_t)nlev * (L - 1) : 0, n_cs = polar ? (size_t)nlev * L * 2 : 0;
  const size_t bytes_pol = sizeof(float) * (n_thr + n_cs);
  // query-prep GEMM operand [Pi; S] (prod mode, d <= 256): (d + m) / 16 row
  // tiles x dpad / 32 column blocks of 64 lane fragments, hi and lo
  const bool pq = mode == TQ_MODE_PROD && d <= 256;
  const size_t pq_tiles = pq ? (size_t)(d + m + 15) / 16 : 0, npq = pq_tiles * (dpad / 32) * 64;
  const size_t off_pq = (bytes_f32 + 255) / 256 * 256 + bytes_fr + (bytes_pol + 255) / 256 * 256;
  const size_t total = off_pq + sizeof(Frag) * 3 * npq;
  std::vector<uint8_t> host(total, 0);
  float *Pi32 = reinterpret_cast<float *>(host.data());
  float *PiT32 = Pi32 + (size_t)d * d;
  float *S32 = PiT32 + (size_t)d * d;
  float *ST32 = S32 + (size_t)m * d;
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) {
      Pi32[(size_t)i * d + j] = (float)hp.Pi[(size_t)i * d + j];
      PiT32[(size_t)j * d + i] = (float)hp.Pi[(size_t)i * d + j];
    }
  for (int i = 0; i < m; ++i)
    for (int j = 0; j < d; ++j) {
      S32[(size_t)i * d + j] = (float)hp.S[(size_t)i * d + j];
      ST32[(size_t)j * m + i] = (float)hp.S[(size_t)i * d + j];
    }
  Frag *fr = reinterpret_cast<Frag *>(host.data() + (bytes_f32 + 255) / 256 * 256);
  const bool plain = dpad > 256 || frac;      // the LDS-staged quantize kernel
  build_frags(hp, dpad, hp.Pi.data(), d, d, false, plain, fr, fr + nfr);
  if (m) {
    std::vector<double> Sp((size_t)m * d, 0.0);   // S' = S Pi^T
    for (int i = 0; i < m; ++i)
      for (int k = 0; k < d; ++k) {
        double acc = 0.0;
        for (int j = 0; j < d; ++j) acc += hp.S[(size_t)i * d + j] * hp.Pi[(size_t)k * d + j];
        Sp[(size_t)i * d + k] = acc;
      }
    build_frags(hp, dpad, Sp.data(), m, d, true, plain, fr + 2 * nfr, fr + 3 * nfr);
  }
  float *pol = reinterpret_cast<float *>(host.data() + (bytes_f32 + 255) / 256 * 256 + bytes_fr);
  if (polar) {
    for (size_t i = 0; i < n_thr; ++i) pol[i] = (float)hp.t[i];
    for (size_t i = 0; i < (size_t)nlev * L; ++i) {
      pol[n_thr + 2 * i] = (float)std::cos(hp.c[i]);
      pol[n_thr + 2 * i + 1] = (float)std::sin(hp.c[i]);
    }
  }
  if (pq) {
    Frag *ph = reinterpret_cast<Frag *>(host.data() + off_pq), *pm = ph + npq, *pl = ph + 2 * npq;
    const int NK = dpad / 32;
    for (size_t u = 0; u < pq_tiles; ++u)
      for (int k = 0; k < NK; ++k)
        for (int l = 0; l < 64; ++l) {
          const int row = 16 * (int)u + l % 16, g = l / 16;
          uint16_t h8[8], m8[8], l8[8];
          for (int e = 0; e < 8; ++e) {
            const int c = 32 * k + 8 * g + e;
            double v = 0.0;
            if (c < d && row < d) v = hp.Pi[(size_t)row * d + c];
            else if (c < d && row < d + m) v = hp.S[(size_t)(row - d) * d + c];
            // three parts: hi = bf16(v), mid = bf16(v - hi), lo = bf16(v - hi - mid)
            h8[e] = bf16_rne((float)v);
            const double r1 = v - (double)bf16_to_f(h8[e]);
            m8[e] = bf16_rne((float)r1);
            l8[e] = bf16_rne((float)(r1 - (double)bf16_to_f(m8[e])));
          }
          Frag fh, fm, fl;
          for (int i = 0; i < 4; ++i) {
            fh.v[i] = (uint32_t)h8[2 * i] | ((uint32_t)h8[2 * i + 1] << 16);
            fm.v[i] = (uint32_t)m8[2 * i] | ((uint32_t)m8[2 * i + 1] << 16);
            fl.v[i] = (uint32_t)l8[2 * i] | ((uint32_t)l8[2 * i + 1] << 16);
          }
          ph[(u * NK + k) * 64 + l] = fh;
          pm[(u * NK + k) * 64 + l] = fm;
          pl[(u * NK + k) * 64 + l] = fl;
        }
  }
  if (hipMalloc(&ctx->dmem, total) != hipSuccess) {
    (void)hipGetLastError();
    delete ctx;
    return TQ_ENOMEM;
  }
  if (hipMemcpy(ctx->dmem, host.data(), total, hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(ctx->dmem);
    delete ctx;
    return TQ_EHIP;
  }
  uint8_t *base = reinterpret_cast<uint8_t *>(ctx->dmem);
  ctx->Pi32 = reinterpret_cast<float *>(base);
  ctx->PiT32 = ctx->Pi32 + (size_t)d * d;
  ctx->S32 = ctx->PiT32 + (size_t)d * d;
  ctx->ST32 = ctx->S32 + (size_t)m * d;
  Frag *dfr = reinterpret_cast<Frag *>(base + (bytes_f32 + 255) / 256 * 256);
  ctx->PiA_hi = dfr;
  ctx->PiA_lo = dfr + nfr;
  if (m) {
    ctx->S2A_hi = dfr + 2 * nfr;
    ctx->S2A_lo = dfr + 3 * nfr;
  }
  if (polar) {
    ctx->polar_thr = reinterpret_cast<float *>(base + (bytes_f32 + 255) / 256 * 256 + bytes_fr);
    ctx->polar_cs = ctx->polar_thr + n_thr;
  }
  if (pq) {
    ctx->PqH = reinterpret_cast<Frag *>(base + off_pq);
    ctx->npq = npq;
  }
  // the static scratch buffer of this device is located once, at init
  if (tq::scratch_attach(ctx->device) == nullptr) {
    (void)hipFree(ctx->dmem);
    delete ctx;
    return TQ_EHIP;
  }
  *out = ctx;
  return TQ_OK;
}

}  // namespace

namespace tq {

// Argument checks of tq_scores apart from its workspace (shared with the
// static-scratch variant).  TQ_OK with G == 0 or T == 0 means nothing to do.
int check_scores_call(const tq_ctx *ctx, const float *q, int64_t G, int qpg, int64_t T, int64_t ldk,
                      const uint8_t *codes, const uint8_t *signs, const float *norms,
                      const float *rnorms, const float *logits) {
  if (!ctx || !scoring_mode(ctx)) return TQ_EINVAL;
  if (G < 0 || T < 0 || ldk < T || qpg < 1 || qpg > TQ_MAX_QPG_SCORES) return TQ_EINVAL;
  if (G == 0 || T == 0) return TQ_OK;
  if (!q || !codes || !signs || !norms || !rnorms || !logits) return TQ_EINVAL;
  if (!aligned(codes, 16) || !aligned(signs, 16) || !aligned(norms, 4) || !aligned(rnorms, 4) ||
      !aligned(q, 4) || !aligned(logits, 4))
    return TQ_EINVAL;
  return current_device_matches(ctx);
}

}  // namespace tq

extern "C" {

int tq_init(int d, int bits, uint64_t seed, tq_ctx **out) {
  return make_ctx(d, bits, seed, TQ_MODE_PROD, out);
}

int tq_init_mse(int d, int bits, uint64_t seed, tq_ctx **out) {
  return make_ctx(d, bits, seed, TQ_MODE_MSE, out);
}

int tq_init_polar(int d, int bits, uint64_t seed, tq_ctx **out) {
  return make_ctx(d, bits, seed, TQ_MODE_POLAR, out);
}

int tq_init_frac(int d, int half_bits, uint64_t seed, tq_ctx **out) {
  return make_ctx(d, half_bits, seed, TQ_MODE_FRAC, out);
}

int tq_polar_codebook(int d, int bits, double *c, double *t) {
  tq::HostParams hp;
  const int st = tq::build_host_params(d, bits, 0, TQ_MODE_POLAR, hp);
  if (st != TQ_OK) return st;
  if (c) std::memcpy(c, hp.c.data(), hp.c.size() * sizeof(double));
  if (t) std::memcpy(t, hp.t.data(), hp.t.size() * sizeof(double));
  return TQ_OK;
}

void tq_free(tq_ctx *ctx) {
  if (!ctx) return;
  if (ctx->dmem) (void)hipFree(ctx->dmem);
  delete ctx;
}

int tq_layout(const tq_ctx *ctx, tq_layout_t *out) {
  if (!ctx || !out) return TQ_EINVAL;
  out->d = ctx->hp.d;
  out->m = ctx->hp.m;
  out->bits = ctx->hp.bits;
  out->code_bits = ctx->hp.w;
  out->levels = ctx->hp.levels;
  out->code_bytes = ctx->code_bytes;
  out->sign_bytes = ctx->sign_bytes;
  out->mode = ctx->hp.mode;
  return TQ_OK;
}

int tq_get_params(const tq_ctx *ctx, double *Pi, double *S, double *c, double *t) {
  if (!ctx) return TQ_EINVAL;
  const tq::HostParams &hp = ctx->hp;
  if (Pi) std::memcpy(Pi, hp.Pi.data(), hp.Pi.size() * sizeof(double));
  if (S && hp.m) std::memcpy(S, hp.S.data(), hp.S.size() * sizeof(double));
  if (c) {
    std::memcpy(c, hp.c.data(), hp.c.size() * sizeof(double));
    if (!hp.c2.empty()) std::memcpy(c + hp.c.size(), hp.c2.data(), hp.c2.size() * sizeof(double));
  }
  if (t) {
    std::memcpy(t, hp.t.data(), hp.t.size() * sizeof(double));
    if (!hp.t2.empty()) std::memcpy(t + hp.t.size(), hp.t2.data(), hp.t2.size() * sizeof(double));
  }
  return TQ_OK;
}

int tq_quantize(const tq_ctx *ctx, const void *x, int dtype, int64_t n, int64_t ldx,
                int64_t ldr, uint8_t *codes, uint8_t *signs, float *norms, float *rnorms,
                hipStream_t stream) {
  if (!ctx || n < 0 || ldr < 1) return TQ_EINVAL;
  if (dtype != TQ_F32 && dtype != TQ_BF16) return TQ_EINVAL;
  const bool prod = ctx->hp.mode == TQ_MODE_PROD || ctx->hp.mode == TQ_MODE_FRAC;
  if (n == 0) return TQ_OK;
  if (!x || !codes || !norms) return TQ_EINVAL;
  if (prod ? (!signs || !rnorms) : (signs || rnorms)) return TQ_EINVAL;
  const bool polar = ctx->hp.mode == TQ_MODE_POLAR;
  if (ldx < ctx->hp.d) return TQ_EINVAL;
  if (dtype == TQ_BF16 ? (ldx % 8) : (ldx % 4)) return TQ_EINVAL;
  // fractional-width records are a multiple of 8 bytes, written as 32-bit
  // words: a record slot of a cache is aligned to 8 bytes only
  if (!aligned(x, 16) || !aligned(codes, ctx->frac ? 4 : 16) || (signs && !aligned(signs, 16)) ||
      !aligned(norms, 4) || (rnorms && !aligned(rnorms, 4)))
    return TQ_EINVAL;
  const int st = current_device_matches(ctx);
  if (st != TQ_OK) return st;
  if (polar) return tq::launch_polar_quantize(ctx, x, dtype, n, ldx, ldr, codes, norms, stream);
  return tq::launch_quantize(ctx, x, dtype, n, ldx, ldr, codes, signs, norms, rnorms, stream);
}

int tq_workspace_size(const tq_ctx *ctx, int op, int64_t a, int64_t b, int64_t c, size_t *bytes) {
  if (!ctx || !bytes || a < 0 || b < 0 || c < 0) return TQ_EINVAL;
  switch (op) {
    case TQ_OP_SCORES:
      if (!scoring_mode(ctx) || b < 1 || b > TQ_MAX_QPG_SCORES) return TQ_EINVAL;
      *bytes = tq::scores_ws_bytes(ctx, a, (int)b);
      return TQ_OK;
    case TQ_OP_ATTEND:
      if (ctx->hp.mode != TQ_MODE_PROD || b < 1 || b > TQ_MAX_QPG) return TQ_EINVAL;
      *bytes = tq::attend_ws_bytes(ctx, a, (int)b, c);
      return TQ_OK;
    case TQ_OP_TOPK:
      if (ctx->hp.mode != TQ_MODE_PROD || c < 1 || c > TQ_MAX_TOPK) return TQ_EINVAL;
      *bytes = tq::topk_ws_bytes(ctx, a, b, (int)c);
      return TQ_OK;
    default:
      return TQ_EINVAL;
  }
}

int tq_scores(const tq_ctx *ctx, const float *q, int64_t G, int qpg, int64_t T, int64_t ldk,
              const uint8_t *codes, const uint8_t *signs, const float *norms,
              const float *rnorms, float *logits, void *ws, size_t ws_bytes,
              hipStream_t stream) {
  int st = tq::check_scores_call(ctx, q, G, qpg, T, ldk, codes, signs, norms, rnorms, logits);
  if (st != TQ_OK || G == 0 || T == 0) return st;
  if (!ws || !aligned(ws, 16)) return TQ_EINVAL;
  if (ws_bytes < tq::scores_ws_bytes(ctx, G, qpg)) return TQ_EINVAL;
  return tq::launch_scores(ctx, q, G, qpg, T, ldk, codes, signs, norms, rnorms, logits, ws, stream);
}

int tq_prep_queries(const tq_ctx *ctx, const float *q, int64_t G, int qpg, void *ws,
                    size_t ws_bytes, hipStream_t stream) {
  if (!ctx || !scoring_mode(ctx)) return TQ_EINVAL;
  if (G < 0 || qpg < 1 || qpg > TQ_MAX_QPG_SCORES) return TQ_EINVAL;
  if (G == 0) return TQ_OK;
  if (!q || !ws || !aligned(q, 4) || !aligned(ws, 16)) return TQ_EINVAL;
  if (ws_bytes < tq::scores_ws_bytes(ctx, G, qpg)) return TQ_EINVAL;
  const int st = current_device_matches(ctx);
  if (st != TQ_OK) return st;
  return tq::launch_prep_queries(ctx, q, G, qpg, ws, stream);
}

int tq_scores_prepared(const tq_ctx *ctx, const void *ws, size_t ws_bytes, int64_t G, int qpg,
                       int64_t T, int64_t ldk, const uint8_t *codes, const uint8_t *signs,
                       const float *norms, const float *rnorms, float *logits,
                       hipStream_t stream) {
  return tq_scores_prepared_timed(ctx, ws, ws_bytes, G, qpg, T, ldk, codes, signs, norms, rnorms, logits,
                                  stream, nullptr, nullptr);
}

int tq_scores_prepared_timed(const tq_ctx *ctx, const void *ws, size_t ws_bytes, int64_t G, int qpg,
                             int64_t T, int64_t ldk, const uint8_t *codes, const uint8_t *signs,
                             const float *norms, const float *rnorms, float *logits,
                             hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (!ctx || !scoring_mode(ctx)) return TQ_EINVAL;
  if (G < 0 || T < 0 || ldk < T || qpg < 1 || qpg > TQ_MAX_QPG_SCORES) return TQ_EINVAL;
  if (G == 0 || T == 0) return TQ_OK;
  if (!ws || !codes || !signs || !norms || !rnorms || !logits) return TQ_EINVAL;
  if (!aligned(codes, 16) || !aligned(signs, 16) || !aligned(norms, 4) || !aligned(rnorms, 4) ||
      !aligned(logits, 4) || !aligned(ws, 16))
    return TQ_EINVAL;
  if (ws_bytes < tq::scores_ws_bytes(ctx, G, qpg)) return TQ_EINVAL;
  const int st = current_device_matches(ctx);
  if (st != TQ_OK) return st;
  return tq::launch_scores_prepared(ctx, ws, G, qpg, T, ldk, codes, signs, norms, rnorms, logits,
                                    stream, start, stop);
}

int tq_softmax(const float *logits, int64_t rows, int64_t T, float scale, float *probs,
               hipStream_t stream) {
  if (rows < 0 || T < 0) return TQ_EINVAL;
  if (rows == 0 || T == 0) return TQ_OK;
  if (!logits || !probs || !aligned(logits, 4) || !aligned(probs, 4)) return TQ_EINVAL;
  if (!std::isfinite(scale)) return TQ_EINVAL;
  return tq::launch_softmax(logits, rows, T, scale, probs, stream);
}

int tq_attend(const tq_ctx *kctx, const tq_ctx *vctx, const float *q, int64_t G, int qpg,
              int64_t T, int64_t ldk, const uint8_t *kcodes, const uint8_t *ksigns,
              const float *knorms, const float *krnorms, const uint8_t *vcodes,
              const float *vnorms, float scale, float *logits, float *probs, float *out,
              void *ws, size_t ws_bytes, hipStream_t stream) {
  if (!kctx || !vctx || kctx->hp.mode != TQ_MODE_PROD || vctx->hp.mode != TQ_MODE_MSE)
    return TQ_EINVAL;
  if (kctx->hp.d != vctx->hp.d) return TQ_EINVAL;
  if (G < 0 || T < 1 || ldk < T || qpg < 1 || qpg > TQ_MAX_QPG) return TQ_EINVAL;
  if (G == 0) return TQ_OK;
  if (!q || !kcodes || !ksigns || !knorms || !krnorms || !vcodes || !vnorms || !out || !ws)
    return TQ_EINVAL;
  if (!aligned(kcodes, 16) || !aligned(ksigns, 16) || !aligned(vcodes, 16) || !aligned(ws, 16) ||
      !aligned(knorms, 4) || !aligned(krnorms, 4) || !aligned(vnorms, 4) || !aligned(q, 4) ||
      !aligned(out, 4) || (logits && !aligned(logits, 4)) || (probs && !aligned(probs, 4)))
    return TQ_EINVAL;
  if (!std::isfinite(scale)) return TQ_EINVAL;
  if (ws_bytes < tq::attend_ws_bytes(kctx, G, qpg, T)) return TQ_EINVAL;
  const int st = current_device_matches(kctx);
  if (st != TQ_OK) return st;
  if (vctx->device != kctx->device) return TQ_EINVAL;
  return tq::launch_attend(kctx, vctx, q, G, qpg, T, ldk, kcodes, ksigns, knorms, krnorms, vcodes,
                           vnorms, scale, logits, probs, out, ws, stream);
}

namespace {

// Checks shared by the decode entry points (vctx may be null: keys only).
int check_decode(const tq_ctx *kctx, const tq_ctx *vctx, const float *q, int64_t G, int qpg,
                 const void *new_k, const void *new_v, int dtype, int64_t ldx, int64_t pos,
                 int64_t ldk, const uint8_t *kcodes, const uint8_t *ksigns, const float *knorms,
                 const float *krnorms, const uint8_t *vcodes, const float *vnorms, const void *ws) {
  if (!kctx || kctx->hp.mode != TQ_MODE_PROD) return TQ_EINVAL;
  if (vctx && (vctx->hp.mode != TQ_MODE_MSE || vctx->hp.d != kctx->hp.d)) return TQ_EINVAL;
  const int d = kctx->hp.d;
  if (G < 0 || qpg < 1 || qpg > TQ_MAX_QPG || pos < 0 || ldk < pos + 1) return TQ_EINVAL;
  if (dtype != TQ_F32 && dtype != TQ_BF16) return TQ_EINVAL;
  if (ldx < d || (dtype == TQ_BF16 ? (ldx % 8) : (ldx % 4))) return TQ_EINVAL;
  if (!q || !new_k || !kcodes || !ksigns || !knorms || !krnorms || !ws) return TQ_EINVAL;
  if (vctx && (!new_v || !vcodes || !vnorms)) return TQ_EINVAL;
  if (!aligned(new_k, 16) || !aligned(kcodes, 16) || !aligned(ksigns, 16) || !aligned(ws, 16) ||
      !aligned(knorms, 4) || !aligned(krnorms, 4) || !aligned(q, 4))
    return TQ_EINVAL;
  if (vctx && (!aligned(new_v, 16) || !aligned(vcodes, 16) || !aligned(vnorms, 4))) return TQ_EINVAL;
  int st = current_device_matches(kctx);
  if (st != TQ_OK) return st;
  if (vctx && vctx->device != kctx->device) return TQ_EINVAL;
  if (G * ((qpg + 3) / 4) > 65535) return TQ_ENOTSUP;
  return TQ_OK;
}

// Append + query prep: one fused launch where the library has one, else the
// quantize and prep launches in turn (same results).
int decode_prep(const tq_ctx *kctx, const tq_ctx *vctx, const float *q, int64_t G, int qpg,
                const void *new_k, const void *new_v, int dtype, int64_t ldx, int64_t pos, int64_t ldk,
                uint8_t *kcodes, uint8_t *ksigns, float *knorms, float *krnorms, uint8_t *vcodes,
                float *vnorms, void *ws, hipStream_t stream) {
  int st = tq::launch_decode_prep(kctx, vctx, q, G, qpg, new_k, new_v, dtype, ldx, pos, ldk, kcodes,
                                  ksigns, knorms, krnorms, vcodes, vnorms, ws, stream);
  if (st != TQ_ENOTSUP) return st;
  st = tq::launch_quantize(kctx, new_k, dtype, G, ldx, ldk, kcodes + pos * kctx->code_bytes,
                           ksigns + pos * kctx->sign_bytes, knorms + pos, krnorms + pos, stream);
  if (st != TQ_OK) return st;
  if (vctx) {
    st = tq::launch_quantize(vctx, new_v, dtype, G, ldx, ldk, vcodes + pos * vctx->code_bytes, nullptr,
                             vnorms + pos, nullptr, stream);
    if (st != TQ_OK) return st;
  }
  return tq::launch_prep_queries(kctx, q, G, qpg, ws, stream);
}

}  // namespace

int tq_decode_prep(const tq_ctx *kctx, const tq_ctx *vctx, const float *q, int64_t G, int qpg,
                   const void *new_k, const void *new_v, int dtype, int64_t ldx, int64_t pos,
                   int64_t ldk, uint8_t *kcodes, uint8_t *ksigns, float *knorms, float *krnorms,
                   uint8_t *vcodes, float *vnorms, void *ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_decode(kctx, vctx, q, G, qpg, new_k, new_v, dtype, ldx, pos, ldk, kcodes, ksigns,
                        knorms, krnorms, vcodes, vnorms, ws);
  if (st != TQ_OK) return st;
  if (G == 0) return TQ_OK;
  if (ws_bytes < tq::scores_ws_bytes(kctx, G, qpg)) return TQ_EINVAL;
  return decode_prep(kctx, vctx, q, G, qpg, new_k, new_v, dtype, ldx, pos, ldk, kcodes, ksigns, knorms,
                     krnorms, vcodes, vnorms, ws, stream);
}

int tq_decode_step(const tq_ctx *kctx, const tq_ctx *vctx, const float *q, int64_t G, int qpg,
                   const void *new_k, const void *new_v, int dtype, int64_t ldx, int64_t pos,
                   int64_t ldk, uint8_t *kcodes, uint8_t *ksigns, float *knorms, float *krnorms,
                   uint8_t *vcodes, float *vnorms, float scale, float *logits, float *probs,
                   float *out, void *ws, size_t ws_bytes, hipStream_t stream) {
  // everything is checked before the first launch: on error nothing is written
  if (!vctx) return TQ_EINVAL;
  int st = check_decode(kctx, vctx, q, G, qpg, new_k, new_v, dtype, ldx, pos, ldk, kcodes, ksigns,
                        knorms, krnorms, vcodes, vnorms, ws);
  if (st != TQ_OK) return st;
  if (G == 0) return TQ_OK;
  if (!out || !aligned(out, 4) || (probs && !logits) || (logits && !aligned(logits, 4)) ||
      (probs && !aligned(probs, 4)) || !std::isfinite(scale))
    return TQ_EINVAL;
  const int64_t T = pos + 1;
  if (ws_bytes < tq::attend_ws_bytes(kctx, G, qpg, T)) return TQ_EINVAL;
  st = tq::check_attend(kctx, vctx, G, qpg, T, ldk, probs != nullptr);
  if (st != TQ_OK) return st;
  // 1-2: the new key and value of every group into slot pos, the queries
  // prepared into the front of ws (the attention workspace starts with them)
  st = decode_prep(kctx, vctx, q, G, qpg, new_k, new_v, dtype, ldx, pos, ldk, kcodes, ksigns, knorms,
                   krnorms, vcodes, vnorms, ws, stream);
  if (st != TQ_OK) return st;
  // 3: attention over tokens 0..pos
  return tq::launch_attend(kctx, vctx, q, G, qpg, T, ldk, kcodes, ksigns, knorms, krnorms, vcodes,
                           vnorms, scale, logits, probs, out, ws, stream, true);
}

int tq_dequant(const tq_ctx *ctx, const uint8_t *codes, const uint8_t *signs, const float *norms,
               const float *rnorms, int64_t n, float *out, hipStream_t stream) {
  if (!ctx || n < 0) return TQ_EINVAL;
  if (n == 0) return TQ_OK;
  const bool prod = scoring_mode(ctx);
  if (!codes || !norms || !out || (prod && (!signs || !rnorms))) return TQ_EINVAL;
  if (!aligned(codes, 16) || (prod && !aligned(signs, 16)) || !aligned(norms, 4) || !aligned(out, 4))
    return TQ_EINVAL;
  const int st = current_device_matches(ctx);
  if (st != TQ_OK) return st;
  return tq::launch_dequant(ctx, codes, prod ? signs : nullptr, norms, prod ? rnorms : nullptr, n,
                            out, stream);
}

int tq_topk(const tq_ctx *ctx, const float *q, int64_t nq, int64_t n, const uint8_t *codes,
            const uint8_t *signs, const float *norms, const float *rnorms, int k, int64_t *ids,
            float *scores, void *ws, size_t ws_bytes, hipStream_t stream) {
  if (!ctx || ctx->hp.mode != TQ_MODE_PROD) return TQ_EINVAL;
  if (nq < 0 || n < 1 || k < 1 || k > TQ_MAX_TOPK || k > n) return TQ_EINVAL;
  if (nq == 0) return TQ_OK;
  if (!q || !codes || !signs || !norms || !rnorms || !ids || !scores || !ws) return TQ_EINVAL;
  if (!aligned(codes, 16) || !aligned(signs, 16) || !aligned(ws, 16) || !aligned(ids, 8) ||
      !aligned(scores, 4) || !aligned(q, 4) || !aligned(norms, 4) || !aligned(rnorms, 4))
    return TQ_EINVAL;
  if (ws_bytes < tq::topk_ws_bytes(ctx, nq, n, k)) return TQ_EINVAL;
  const int st = current_device_matches(ctx);
  if (st != TQ_OK) return st;
  return tq::launch_topk(ctx, q, nq, n, codes, signs, norms, rnorms, k, ids, scores, ws, stream);
}

const char *tq_strerror(int status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_EINVAL: return "invalid argument";
    case TQ_ENOTSUP: return "not supported";
    case TQ_ENOMEM: return "out of memory";
    case TQ_EHIP: return "HIP runtime error";
    case TQ_ESCRATCH: return "request needs more memory than the library's static scratch buffer holds";
    default: return "unknown status";
  }
}

}  // extern "C"
