// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

#include "../../include/tq.h"

namespace tq {

struct HostParams {
  int d = 0, m = 0, bits = 0, w = 0, levels = 0, mode = 0;
  int w2 = 0;              // fractional mode: code bits of the second half (w: the first)
  uint64_t seed = 0;
  std::vector<double> Pi;  // [d][d] row-major
  std::vector<double> S;   // [m][d] row-major
  std::vector<double> c;   // [levels] ascending, for N(0, 1/d); polar mode:
                           // [log2 d][levels], the angle codebook of every level
  std::vector<double> t;   // [levels-1] ascending; polar mode: [log2 d][levels-1]
  std::vector<double> c2, t2;   // fractional mode: the second half's codebook
};

int build_host_params(int d, int bits, uint64_t seed, int mode, HostParams &hp);
void lloyd_max_unit_gaussian(int L, std::vector<double> &c, std::vector<double> &t);
void lloyd_max_polar_angle(int level, int L, std::vector<double> &c, std::vector<double> &t);

// 16-byte MFMA operand fragment (8 x bf16 or 16 x int8 per lane).
struct alignas(16) Frag {
  uint32_t v[4];
};

}  // namespace tq

// The context.  Immutable after tq_init.
struct tq_ctx {
  tq::HostParams hp;
  int device = 0;
  int cus = 256;       // compute units of that device (grid sizing)
  int dpad = 0;        // d rounded up to the quantize kernel's tile (32/64/128/256, then 32 k)
  int code_bytes = 0;
  int sign_bytes = 0;
  float alpha = 0.f;   // sqrt(pi/2) / m
  float cpos[8] = {};  // positive centroids c_{L/2 + j}
  float tpos[8] = {};  // positive thresholds t_{L/2 + j}
  float cf[16] = {};   // all centroids, fp32
  float basis[4] = {}; // odd-basis coefficients of the codebook (see tq_scores.hip)
  float vbasis[8] = {}; // all odd monomials of up to 4 code bits: w singles, then triples
  // fractional mode (TQ_MODE_FRAC): the second half's codebook
  int frac = 0;
  float cpos2[8] = {}, tpos2[8] = {}, cf2[16] = {}, basis2[4] = {};
  // record words per lane group of the scoring kernels (code_bytes / 16, or
  // the first half's w d/128 planar words in fractional mode)
  int cw16 = 0;
  // device constants (one allocation owned by the context)
  void *dmem = nullptr;
  float *Pi32 = nullptr;    // [d][d] row-major
  float *PiT32 = nullptr;   // [d][d] = Pi^T row-major
  float *S32 = nullptr;     // [m][d]
  float *ST32 = nullptr;    // [d][m] = S^T
  tq::Frag *PiA_hi = nullptr, *PiA_lo = nullptr;   // quantize GEMM-1 operand fragments
  tq::Frag *S2A_hi = nullptr, *S2A_lo = nullptr;   // quantize GEMM-2 operand fragments
  // query-prep GEMM operand: [Pi; S] (rows 16 u + r, columns 32 k + 8 g + e)
  // in three bf16 parts (hi, mid, lo: npq fragments each, consecutive), prod
  // mode with d <= 256
  tq::Frag *PqH = nullptr;
  size_t npq = 0;
  float *polar_thr = nullptr;   // polar mode: angle thresholds [log2 d][levels - 1]
  float *polar_cs = nullptr;    // polar mode: (cos, sin) of angle centroids [log2 d][levels][2]
};

namespace tq {

// kernel launchers (return TQ_OK / TQ_EHIP / TQ_ENOTSUP)
int launch_quantize(const tq_ctx *ctx, const void *x, int dtype, int64_t n, int64_t ldx,
                    int64_t ldr, uint8_t *codes, uint8_t *signs, float *norms, float *rnorms,
                    hipStream_t stream);
// vectors longer than 256 coordinates (tq_big.hip)
int launch_quantize_big(const tq_ctx *ctx, const void *x, int dtype, int64_t n, int64_t ldx,
                        int64_t ldr, uint8_t *codes, uint8_t *signs, float *norms, float *rnorms,
                        hipStream_t stream);
int launch_prep_big(const tq_ctx *ctx, const float *q, int64_t groups, int qpg, int hg,
                    int64_t nq_total, uint8_t *ws, hipStream_t stream);
// query prep of many groups as one MFMA GEMM (tq_prep_gemm.hip)
bool prep_gemm_applies(const tq_ctx *ctx, int64_t groups);
int launch_prep_gemm(const tq_ctx *ctx, const float *q, int64_t groups, int qpg, int hg,
                     int64_t nq_total, uint8_t *ws, hipStream_t stream);
int launch_polar_quantize(const tq_ctx *ctx, const void *x, int dtype, int64_t n, int64_t ldx,
                          int64_t ldr, uint8_t *codes, float *norms, hipStream_t stream);
size_t scores_ws_bytes(const tq_ctx *ctx, int64_t G, int qpg);
int launch_scores(const tq_ctx *ctx, const float *q, int64_t G, int qpg, int64_t T, int64_t ldk,
                  const uint8_t *codes, const uint8_t *signs, const float *norms,
                  const float *rnorms, float *logits, void *ws, hipStream_t stream);
int launch_prep_queries(const tq_ctx *ctx, const float *q, int64_t G, int qpg, void *ws,
                        hipStream_t stream);
int launch_scores_prepared(const tq_ctx *ctx, const void *ws, int64_t G, int qpg, int64_t T,
                           int64_t ldk, const uint8_t *codes, const uint8_t *signs,
                           const float *norms, const float *rnorms, float *logits,
                           hipStream_t stream,
                           hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
int launch_softmax(const float *logits, int64_t rows, int64_t T, float scale, float *probs,
                   hipStream_t stream);
int launch_dequant(const tq_ctx *ctx, const uint8_t *codes, const uint8_t *signs,
                   const float *norms, const float *rnorms, int64_t n, float *out,
                   hipStream_t stream);
size_t attend_ws_bytes(const tq_ctx *k, int64_t G, int qpg, int64_t T);
// shape limits of launch_attend (TQ_OK or TQ_ENOTSUP), checked before any launch
int check_attend(const tq_ctx *kc, const tq_ctx *vc, int64_t G, int qpg, int64_t T, int64_t ldk,
                 bool want_probs);
int launch_attend(const tq_ctx *kc, const tq_ctx *vc, const float *q, int64_t G, int qpg,
                  int64_t T, int64_t ldk, const uint8_t *kcodes, const uint8_t *ksigns,
                  const float *knorms, const float *krnorms, const uint8_t *vcodes,
                  const float *vnorms, float scale, float *logits, float *probs, float *out,
                  void *ws, hipStream_t stream, bool prepped = false);
// Append one token per group (keys in kc, values in vc if not null) at record
// g * ldk + pos and prepare the queries into ws, in one launch.  TQ_ENOTSUP
// when the library has no fused kernel for the shapes (the caller then runs
// launch_quantize and the prep apart).
int launch_decode_prep(const tq_ctx *kc, const tq_ctx *vc, const float *q, int64_t G, int qpg,
                       const void *new_k, const void *new_v, int dtype, int64_t ldx, int64_t pos,
                       int64_t ldk, uint8_t *kcodes, uint8_t *ksigns, float *knorms, float *krnorms,
                       uint8_t *vcodes, float *vnorms, void *ws, hipStream_t stream);
size_t topk_ws_bytes(const tq_ctx *ctx, int64_t nq, int64_t n, int k);
int launch_topk(const tq_ctx *ctx, const float *q, int64_t nq, int64_t n, const uint8_t *codes,
                const uint8_t *signs, const float *norms, const float *rnorms, int k,
                int64_t *ids, float *scores, void *ws, hipStream_t stream);

// tq_scores argument checks apart from the workspace (tq_api.cpp)
int check_scores_call(const tq_ctx *ctx, const float *q, int64_t G, int qpg, int64_t T, int64_t ldk,
                      const uint8_t *codes, const uint8_t *signs, const float *norms,
                      const float *rnorms, const float *logits);
// Device address of the static scratch buffer on `device` (tq_static.hip),
// looked up once per device with that device current; nullptr on failure.
void *scratch_attach(int device);

inline int hip_status() { return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP; }

// Lets kernel fn take `bytes` of dynamic LDS (beyond the 64 KB allowed by
// default; a CU has 160 KB).
inline int allow_lds(const void *fn, size_t bytes) {
  if (bytes <= 65536) return TQ_OK;
  if (bytes > 163840) return TQ_ENOTSUP;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) == hipSuccess ? TQ_OK
                                                                                                        : TQ_EHIP;
}

}  // namespace tq
