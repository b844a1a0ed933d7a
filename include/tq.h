/*
 * tq.h -- C ABI of the MI355X (gfx950) TurboQuant hot path.
 *
 * TurboQuant compresses KV-cache keys in two stages and scores them against an
 * uncompressed query:
 *   stage 1: keep the vector length, rotate the unit vector by a seeded random
 *            orthogonal matrix Pi, code each rotated coordinate with a
 *            Max-Lloyd scalar codebook built for N(0, 1/d)
 *            (suzuke blog "turboquant-compressing-ai-consciousness",
 *             section 技術上怎麼做到的, 第一步 and 第二步; xujun.org note 189244,
 *             section 第一步：PolarQuant);
 *   stage 2: project the stage-1 residual with a Gaussian JL matrix S and keep
 *            one sign bit per row (xujun.org note 189244, section 第二步：QJL;
 *            hao.cnyes.com "TurboQuant", heading 1 bit 掃尾);
 *   score:   l = nu * (<Pi q, c[idx]> + alpha * gamma * <S q, 2 bits - 1>),
 *            alpha = sqrt(pi/2) / m, which is unbiased in expectation
 *            (xujun.org note 189244, 第二步：QJL; suzuke blog, 第三步).
 * Nothing is calibrated on data: a context is fixed by (d, bits, seed) alone
 * (xujun.org note 189244, 常见问题 -- data-oblivious).
 *
 * Conventions for every call:
 *   - Returns TQ_OK (0) or a negative TQ_E* code.  Arguments are validated
 *     before anything is launched; on an error no output is touched.
 *     Asynchronous kernel faults surface at the caller's next synchronisation
 *     of `stream`.  No call aborts the process or throws across the ABI.
 *   - Array pointers marked [device] are device memory owned by the caller;
 *     base pointers must be 16-byte aligned.  The library keeps no pointer
 *     after a call returns.  A context owns its device constants until
 *     tq_free().  A context is immutable after init, so concurrent calls on
 *     different streams are safe.
 *   - Compute calls are stream-ordered and asynchronous on `stream` (NULL =
 *     the default stream of the current device), and never allocate: calls
 *     that need scratch memory take a caller workspace sized by
 *     tq_workspace_size().
 *
 * Packed record layout (structure-of-arrays, one record per vector):
 *   codes [n][code_bytes]  prod mode: code i of a vector sits in bits
 *                          [i*w, (i+1)*w) of its record, little-endian, LSB
 *                          first; MSE-only mode: w bit planes of d bits, plane
 *                          p in bytes [p*d/8, (p+1)*d/8) holding bit p of code
 *                          i at bit i of the plane (LSB first); code k selects
 *                          the k-th smallest centroid;
 *   signs [n][sign_bytes]  sign bit j is bit (j & 7) of byte (j >> 3); 1 = +1
 *                          (prod mode only);
 *   norms [n]   float32    nu = |x|_2;
 *   rnorms[n]   float32    gamma = |stage-1 residual of x/nu|_2 (prod only).
 *   code_bytes = roundup16(ceil(d*w/8)), sign_bytes = roundup16(ceil(m/8)),
 *   padding bytes are zero.  A zero vector is stored as zero codes, zero signs,
 *   nu = 0, gamma = 0.  Appending = writing at a record offset.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define TQ_OK        0
#define TQ_EINVAL   (-1)   /* bad dimension, bit width, size, pointer, alignment or mode */
#define TQ_ENOTSUP  (-2)   /* valid request the library does not implement */
#define TQ_ENOMEM   (-3)   /* host or device allocation failed (init only) */
#define TQ_EHIP     (-4)   /* a HIP runtime call or kernel launch failed */
#define TQ_ESCRATCH (-5)   /* the request needs more scratch memory than the
                              library's static buffer (TQ_SCRATCH_BYTES) holds */

/* input element types for tq_quantize */
#define TQ_F32   0
#define TQ_BF16  1

/* modes */
#define TQ_MODE_PROD 0     /* (bits-1)-bit codes + 1-bit QJL sketch, m = d */
#define TQ_MODE_MSE  1     /* bits-bit codes only (no sketch)              */
#define TQ_MODE_POLAR 2    /* bits-bit codes of the recursive polar angles  */
#define TQ_MODE_FRAC  3    /* b = bits/2 (2.5, 3.5): codes of ceil(b)-1 and
                              floor(b)-1 bits on the two halves + 1-bit QJL */

/* ops for tq_workspace_size */
#define TQ_OP_SCORES  1
#define TQ_OP_ATTEND  2
#define TQ_OP_TOPK    3

/* limits of the library */
#define TQ_MAX_D       1024  /* d in [8, 1024], d % 8 == 0 */
#define TQ_MAX_TOPK    1024
#define TQ_MAX_QPG     64    /* query heads per group: attention and decode steps */
#define TQ_MAX_QPG_SCORES 65536  /* queries per group: tq_scores, tq_prep_queries,
                                    tq_scores_prepared (many queries against one key
                                    set, e.g. every position of a prefill); in addition
                                    G * ceil(qpg / 4) <= 65535, else TQ_ENOTSUP */

typedef struct tq_ctx tq_ctx;

typedef struct {
  int d;           /* vector dimension                                  */
  int m;           /* JL rows (= d in prod mode, 0 in mse mode)         */
  int bits;        /* total bits per coordinate requested at init
                      (TQ_MODE_FRAC: twice the bits per coordinate)     */
  int code_bits;   /* w: bits per scalar code (bits-1 prod, bits mse;
                      TQ_MODE_FRAC: of the first half; the second
                      half's codes have w - 1 bits)                     */
  int levels;      /* 2^w codebook entries                              */
  int code_bytes;  /* bytes per code record                             */
  int sign_bytes;  /* bytes per sign record (0 in mse mode)             */
  int mode;        /* TQ_MODE_PROD, _MSE, _POLAR or _FRAC               */
} tq_layout_t;

/* Build a prod-mode context: Pi = Haar(d) as Q diag(sign R_ii) of the QR
 * factorisation of a d x d Gaussian matrix (SplitMix64 sub-stream 0 + Box-
 * Muller), S = m x d Gaussian (sub-stream 1), m = d, and the Lloyd-Max codebook
 * with 2^(bits-1) levels for N(0, 1/d) (suzuke blog, 第一步/第二步; xujun.org
 * note 189244, 第二步：QJL).  d in [8, TQ_MAX_D] with d % 8 == 0; bits in
 * {2,3,4}.  Synchronous; uploads constants to the current device.  *out is
 * written only on success. */
int tq_init(int d, int bits, uint64_t seed, tq_ctx **out);

/* Same, MSE-only mode: 2^bits levels, no sketch; bits in {1,2,3,4}. */
int tq_init_mse(int d, int bits, uint64_t seed, tq_ctx **out);

/* PolarQuant context (MSE-only stage; xujun.org note 189244, 第一步：PolarQuant;
 * suzuke blog, 第二步): y = Pi x / |x| is written in recursive polar
 * coordinates -- level 1 pairs coordinates (2i, 2i+1) into (radius, angle in
 * [0, 2 pi)), every further level pairs two radii into (radius, angle in
 * [0, pi/2]), down to the radius |y| = 1 -- and each of the d - 1 angles takes
 * a bits-bit code from its level's Lloyd-Max codebook (level 1: uniform
 * cells; level l >= 2: the law with sin^2 ~ Beta(k/2, k/2), k = 2^(l-1)).
 * d in {32, 64, 128, 256}, bits in {1,2,3,4}.  Records: d slots of bits bits
 * (code_bytes = roundup16(d bits / 8)) + the float32 length; slots
 * [q d/4, (q+1) d/4) hold the subtree of coordinate quarter q level by level,
 * then a spare slot holding the top angle (q = 0), the level log2(d)-1 angle
 * of quarters 0/1 (q = 1) or 2/3 (q = 2), or zero (q = 3).  Such a context
 * takes tq_quantize (signs and rnorms NULL) and tq_dequant; the estimator
 * calls (tq_scores, tq_attend, tq_topk, decode steps) return TQ_EINVAL. */
int tq_init_polar(int d, int bits, uint64_t seed, tq_ctx **out);

/* Fractional-width context, b = half_bits / 2 bits per coordinate with
 * half_bits in {5, 7} (2.5 and 3.5 bits: suzuke blog, 實際跑出來的數據;
 * xujun.org note 189244, 跑分全面碾压; the pages give no mechanism, and this
 * is the library's reading).  Pi and S as tq_init with the same seed; the
 * rotated coordinates 0 .. d/2-1 take codes of w_hi = ceil(b) - 1 bits, the
 * rest w_lo = floor(b) - 1 bits, each half with the Lloyd-Max codebook for
 * N(0, 1/d) at its width; one QJL sign bit per JL row (m = d) of the stage-1
 * residual over all coordinates, so the estimator keeps its form.  Records:
 * code_bytes = d (w_hi + w_lo) / 16 (no padding), laid out by coordinate
 * quarter: quarter g (coordinates [g d/4, (g+1) d/4)) holds w_g bit planes of
 * d/4 bits, plane p = bit p of the quarter's codes in order (w_g = w_hi for
 * g < 2, else w_lo); sign records, norms and residual norms as tq_init.
 * d in {128, 256}; tq_quantize takes a codes pointer aligned to 4 bytes
 * (a record slot inside a cache).  Such a context takes tq_quantize, tq_dequant and the
 * scoring calls (tq_scores, tq_prep_queries, tq_scores_prepared(_timed),
 * tq_scores_static); tq_attend, tq_topk and the decode steps return
 * TQ_EINVAL. */
int tq_init_frac(int d, int half_bits, uint64_t seed, tq_ctx **out);

/* Host-only: the float64 angle codebooks a PolarQuant context holds, per level
 * l = 1..log2(d): c [log2 d][2^bits] centroids, t [log2 d][2^bits - 1]
 * thresholds (radians).  Either pointer may be NULL. */
int tq_polar_codebook(int d, int bits, double *c, double *t);

/* Release a context (NULL is a no-op). */
void tq_free(tq_ctx *ctx);

/* Record sizes and code parameters of a context. */
int tq_layout(const tq_ctx *ctx, tq_layout_t *out);

/* Host-only: compute the float64 parameters a context would hold, without a
 * GPU.  Pi [d*d] row-major, S [m*d] row-major (prod mode), c [2^w] ascending
 * centroids, t [2^w - 1] ascending thresholds (already scaled by 1/sqrt(d)).
 * Any output pointer may be NULL.  mode = TQ_MODE_PROD, TQ_MODE_MSE or
 * TQ_MODE_FRAC (bits = half_bits; c and t then hold the first half's codebook
 * followed by the second's: 2^w_hi + 2^w_lo centroids, 2^w_hi + 2^w_lo - 2
 * thresholds); else TQ_EINVAL (see tq_polar_codebook for PolarQuant). */
int tq_host_params(int d, int bits, uint64_t seed, int mode,
                   double *Pi, double *S, double *c, double *t);

/* Host copies of a context's float64 parameters (any pointer may be NULL);
 * for a PolarQuant context c and t are the per-level angle codebooks of
 * tq_polar_codebook (log2(d) x 2^bits and log2(d) x (2^bits - 1) doubles);
 * for a fractional-width context both halves' codebooks, as tq_host_params. */
int tq_get_params(const tq_ctx *ctx, double *Pi, double *S, double *c, double *t);

/* Quantize n vectors (online append: any n >= 0).
 *   x      [device] n rows of d elements, row stride ldx elements (ldx >= d;
 *          ldx % 8 == 0 for TQ_BF16, ldx % 4 == 0 for TQ_F32);
 *   dtype  TQ_F32 or TQ_BF16;
 *   ldr    record stride (>= 1): vector i is written to record i * ldr, so a
 *          decode step can append one token to each of n caches laid out
 *          [n][ldr] by passing the record pointers of slot t;
 *   codes  [device] records of code_bytes;  signs [device] records of
 *          sign_bytes (prod), must be NULL in mse mode;  norms [device]
 *          floats;  rnorms [device] floats (prod), NULL in mse mode.
 * Steps per vector: nu = |x|; y = Pi x / nu; idx_i = #{k : t_k < y_i};
 * r = y - c[idx]; gamma = |r|; bit_j = [ (S Pi^T r)_j >= 0 ]
 * (xujun.org note 189244, 第一步 and 第二步; suzuke blog, 第二步 and 第三步). */
int tq_quantize(const tq_ctx *ctx, const void *x, int dtype, int64_t n, int64_t ldx,
                int64_t ldr, uint8_t *codes, uint8_t *signs, float *norms, float *rnorms,
                hipStream_t stream);

/* Workspace bytes needed by an op:
 *   TQ_OP_SCORES: a = G, b = qpg;  TQ_OP_ATTEND: a = G, b = qpg, c = T;
 *   TQ_OP_TOPK:   a = nq, b = n, c = k. */
int tq_workspace_size(const tq_ctx *ctx, int op, int64_t a, int64_t b, int64_t c,
                      size_t *bytes);

/* Asymmetric estimator (hao.cnyes.com "TurboQuant", 1 bit 掃尾: uncompressed
 * query against compressed keys; suzuke blog, 第三步: approximation + residual
 * correction).  GQA: G key groups, qpg query heads per group.
 *   q      [device] float [G][qpg][d];
 *   keys   records [G][ldk] (group g, token t at record g*ldk + t), t < T;
 *   logits [device] float [G][qpg][T]: raw inner-product estimates (no
 *          1/sqrt(d) scaling);
 *   ws     [device] >= tq_workspace_size(TQ_OP_SCORES, G, qpg) bytes.
 * Requires a prod-mode or fractional-width context; T >= 0, ldk >= T,
 * 1 <= qpg <= TQ_MAX_QPG_SCORES
 * (TQ_EINVAL), G * ceil(qpg / 4) <= 65535 (TQ_ENOTSUP).  Queries are scored in
 * blocks of 4 against every key, so a large qpg (all positions of a prefill
 * against the same keys) is one call. */
int tq_scores(const tq_ctx *ctx, const float *q, int64_t G, int qpg, int64_t T, int64_t ldk,
              const uint8_t *codes, const uint8_t *signs, const float *norms,
              const float *rnorms, float *logits, void *ws, size_t ws_bytes,
              hipStream_t stream);

/* The two halves of tq_scores, for callers that prepare the queries apart
 * from scoring (on another stream while the cache is still being appended
 * to, or once for several key sets).
 *
 * tq_prep_queries projects the queries with Pi and S (the query side of the
 * estimator: hao.cnyes.com "TurboQuant", 1 bit 掃尾; suzuke blog, 第三步) and
 * writes, per group and 4-head block, the int8 operand fragments and per-head
 * constants that scoring reads into ws.
 *   q  [device] float [G][qpg][d];
 *   ws [device] >= tq_workspace_size(TQ_OP_SCORES, G, qpg) bytes, written.
 * tq_scores_prepared scores key records against a workspace prepared by
 * tq_prep_queries with the same ctx, G and qpg (read only; it stays valid
 * until the caller overwrites it), with the arguments and results of
 * tq_scores.  tq_scores(...) is tq_prep_queries followed by
 * tq_scores_prepared on the same stream; results are identical. */
int tq_prep_queries(const tq_ctx *ctx, const float *q, int64_t G, int qpg, void *ws,
                    size_t ws_bytes, hipStream_t stream);
int tq_scores_prepared(const tq_ctx *ctx, const void *ws, size_t ws_bytes, int64_t G, int qpg,
                       int64_t T, int64_t ldk, const uint8_t *codes, const uint8_t *signs,
                       const float *norms, const float *rnorms, float *logits,
                       hipStream_t stream);

/* tq_scores_prepared with kernel timing: identical arguments, checks and
 * results; in addition the scores kernel's own dispatch records `start` when
 * it begins and `stop` when it ends (hipExtLaunchKernel), so that
 * hipEventElapsedTime(start, stop) is the kernel's execution time, with no
 * event packets of their own around it on the stream.  start and stop are
 * events the caller created on the ctx's device with timing enabled; either
 * may be NULL.  When G or T is 0 nothing is launched and the events are not
 * touched.  The events stay owned by the caller. */
int tq_scores_prepared_timed(const tq_ctx *ctx, const void *ws, size_t ws_bytes, int64_t G, int qpg,
                             int64_t T, int64_t ldk, const uint8_t *codes, const uint8_t *signs,
                             const float *norms, const float *rnorms, float *logits,
                             hipStream_t stream, hipEvent_t start, hipEvent_t stop);

/* Row softmax of scale * logits: probs[r][t] = exp(s l - max_r) / sum.
 * logits, probs [device] float [rows][T]; probs == logits is allowed. */
int tq_softmax(const float *logits, int64_t rows, int64_t T, float scale, float *probs,
               hipStream_t stream);

/* One fused decode-attention step over a packed KV cache: keys in a prod-mode
 * context kctx, values in an MSE-mode context vctx with the same d
 * (xujun.org note 189244, KV 缓存: both K and V are cached).
 *   out[g][h] = sum_t softmax_t(scale * l[g][h][t]) * vhat[g][t],
 *   vhat = nu_v Pi_v^T c_v[idx_v]  (computed in Pi_v coordinates, rotated
 *   back once per head).
 *   q [device] float [G][qpg][d]; key records [G][ldk]; value records [G][ldk];
 *   logits, probs: optional [device] float [G][qpg][T] outputs (NULL = skip);
 *   out [device] float [G][qpg][d];
 *   ws [device] >= tq_workspace_size(TQ_OP_ATTEND, G, qpg, T). */
int tq_attend(const tq_ctx *kctx, const tq_ctx *vctx, const float *q, int64_t G, int qpg,
              int64_t T, int64_t ldk,
              const uint8_t *kcodes, const uint8_t *ksigns, const float *knorms,
              const float *krnorms, const uint8_t *vcodes, const float *vnorms,
              float scale, float *logits, float *probs, float *out,
              void *ws, size_t ws_bytes, hipStream_t stream);

/* The append + query-prep half of a decode step: the new key of every group
 * (and, if vctx is not NULL, its new value) is quantized into record
 * g*ldk + pos of the caches, and the queries are prepared into ws exactly as
 * tq_prep_queries does (so tq_scores_prepared over T = pos + 1 tokens
 * follows).  For d = 128 and up to 4096 groups the jobs run in one launch
 * (they are independent and each is latency-bound); otherwise in turn.
 * Arguments as in tq_quantize and tq_prep_queries; pos < ldk;
 * ws >= tq_workspace_size(TQ_OP_SCORES, G, qpg).  All checks happen before
 * the first launch. */
int tq_decode_prep(const tq_ctx *kctx, const tq_ctx *vctx, const float *q, int64_t G, int qpg,
                   const void *new_k, const void *new_v, int dtype, int64_t ldx, int64_t pos,
                   int64_t ldk, uint8_t *kcodes, uint8_t *ksigns, float *knorms, float *krnorms,
                   uint8_t *vcodes, float *vnorms, void *ws, size_t ws_bytes, hipStream_t stream);

/* One online decode step (xujun.org note 189244, KV 缓存: every generated
 * token's key and value are compressed as they are produced and appended to
 * the cache): on one stream, with no host synchronisation,
 *   1. the new key of every group, new_k[g] (row stride ldx, fp32 or bf16),
 *      is quantized into key record g*ldk + pos (tq_quantize, kctx);
 *   2. the new value new_v[g] into value record g*ldk + pos (vctx);
 *   3. tq_attend over tokens 0..pos (T = pos + 1) of every group.
 * Steps 1-2 and the query prep of step 3 are tq_decode_prep (one launch for
 * d = 128).
 * Arguments as in tq_quantize and tq_attend; pos < ldk;
 * ws >= tq_workspace_size(TQ_OP_ATTEND, G, qpg, pos + 1) bytes.  All checks
 * happen before the first launch: on error nothing is written. */
int tq_decode_step(const tq_ctx *kctx, const tq_ctx *vctx, const float *q, int64_t G, int qpg,
                   const void *new_k, const void *new_v, int dtype, int64_t ldx, int64_t pos,
                   int64_t ldk, uint8_t *kcodes, uint8_t *ksigns, float *knorms, float *krnorms,
                   uint8_t *vcodes, float *vnorms, float scale, float *logits, float *probs,
                   float *out, void *ws, size_t ws_bytes, hipStream_t stream);

/* Reconstruct n vectors: prod x_hat = nu (Pi^T c[idx] + alpha gamma S^T (2 bits - 1)),
 * mse x_hat = nu Pi^T c[idx] (suzuke blog, 第三步).  out [device] float [n][d].
 * signs/rnorms are ignored (may be NULL) in mse mode. */
int tq_dequant(const tq_ctx *ctx, const uint8_t *codes, const uint8_t *signs,
               const float *norms, const float *rnorms, int64_t n, float *out,
               hipStream_t stream);

/* Inner-product top-k search over n packed database vectors (xujun.org note
 * 189244, 常见问题: vector search, recall 1@k).
 *   q [device] float [nq][d]; database records [n];
 *   ids [device] int64 [nq][k], scores [device] float [nq][k], ordered by
 *   (score descending, id ascending);  1 <= k <= min(n, TQ_MAX_TOPK);
 *   ws [device] >= tq_workspace_size(TQ_OP_TOPK, nq, n, k). */
int tq_topk(const tq_ctx *ctx, const float *q, int64_t nq, int64_t n,
            const uint8_t *codes, const uint8_t *signs, const float *norms,
            const float *rnorms, int k, int64_t *ids, float *scores,
            void *ws, size_t ws_bytes, hipStream_t stream);

/* tq_scores for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments, checks, kernels and results as tq_scores, but the prepared
 * queries live in a static device buffer of TQ_SCRATCH_BYTES that the library
 * holds on each GPU it runs on until the process ends, so the call takes no
 * workspace and allocates nothing.  Requests whose prepared queries,
 * tq_workspace_size(TQ_OP_SCORES, G, qpg), exceed TQ_SCRATCH_BYTES return
 * TQ_ESCRATCH before anything is launched.  Every call on one GPU shares that
 * GPU's buffer: calls that overlap in time on one GPU (on different streams
 * or from different threads) race and must be serialised by the caller. */
#define TQ_SCRATCH_BYTES (16 << 20)
int tq_scores_static(const tq_ctx *ctx, const float *q, int64_t G, int qpg, int64_t T, int64_t ldk,
                     const uint8_t *codes, const uint8_t *signs, const float *norms,
                     const float *rnorms, float *logits, hipStream_t stream);

/* Static string for a status code. */
const char *tq_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* TQ_H */
