// Asymmetric estimator over packed keys, on int8 MFMA.
//
// The estimate for query q and packed key (idx, bits, nu, gamma) is the stage-1
// approximation plus the QJL residual correction (suzuke blog
// "turboquant-compressing-ai-consciousness", 技術上怎麼做到的 / 第三步;
// xujun.org note 189244, 第二步：QJL; hao.cnyes.com "TurboQuant", 1 bit 掃尾):
//   l = nu * ( P + alpha * gamma * Q ),
//   P = <Pi q, c[idx]>,   Q = <S q, 2 bits - 1>,   alpha = sqrt(pi/2)/m.
//
// Formulation used here.  The Lloyd-Max codebook is antisymmetric
// (c[L-1-k] = -c[k]), so with sign variables s_p = 2 beta_p - 1 of the code
// bits beta_p the centroid is an odd multilinear polynomial:
//   w = 1: c = A0 s0;   w = 2: c = A0 s0 + A1 s1;
//   w = 3: c = A0 s0 + A1 s1 + A2 s2 + A3 s0 s1 s2,  with s0 s1 s2 = 2 pi - 1
// where pi is the parity of the three code bits.  Hence P and Q are weighted
// sums of single bits of the packed record:
//   P = sum_bits 2 A_p q_rot[i] beta - (sum_p A_p) sum_i q_rot[i]  (+ parity term),
//   Q = sum_j 2 q_s[j] bit_j - sum_j q_s[j].
// A bit sum is an int8 matrix product: the B operand of
// v_mfma_i32_16x16x64_i8 is built from a packed 32-bit word W as
// W & (0x01010101 << j), i.e. bit j of each byte (value 2^j, or -128 for j = 7),
// one VALU op per 4 bits.  The A operand (16 rows = 4 query heads x 4 base-128
// digits) carries the coefficients as a fixed-point expansion whose scale
// absorbs the 2^j; accumulation is exact in int32, and the digits are
// recombined in fp32.  Four digits keep the coefficient error below ~2.5e-7 of
// the largest coefficient.  A query-prep kernel builds these A fragments once
// per (KV group, head group) into the caller's workspace.
#include "tq_score_core.h"

namespace tq {
namespace {

constexpr int PREP_THREADS = 256;

#ifndef TQ_SCORES_PREFETCH
#define TQ_SCORES_PREFETCH 1
#endif
#ifndef TQ_SCORES_WAVES
#define TQ_SCORES_WAVES 32768
#endif

struct PrepArgs {
  const float *q;      // [G][qpg][d]
  const float *PiT;    // [d][d]
  const float *ST;     // [d][m]
  uint8_t *ws;
  int64_t nq_total;    // queries beyond this flat index are zero
  int d, m, w, qpg, hg, cb, sb, nm;
  float basis[4];
};

// Build the int8 A fragments and per-head constants for one (group, head group).
// Pi^T and S^T are staged through LDS in row chunks with 16-byte cooperative
// loads, so the query products do not wait on one global load at a time.
constexpr int PREP_STAGE_FLOATS = 8192;   // 32 KB staging buffer

// out[hh][i] = sum_j MT[j][i] * qv[hh][j]  for i < cols (MT row-major [d][cols])
__device__ inline void apply_T(const float *MT, int d, int cols, const float (*qv)[TQ_MAX_D],
                               float (*out)[TQ_MAX_D], float *stage) {
  const int tid = threadIdx.x;
  const int rows_per = PREP_STAGE_FLOATS / cols;           // rows of MT per chunk
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < d; j0 += rows_per) {
    const int nr = min(rows_per, d - j0);
    const int n4 = nr * cols / 4;                           // cols % 8 == 0
    const float4 *src = reinterpret_cast<const float4 *>(MT + (int64_t)j0 * cols);
    __syncthreads();
    for (int base = 0; base < n4; base += 8 * PREP_THREADS) {   // 8 loads in flight per thread
      float4 tmp[8];
#pragma unroll
      for (int b = 0; b < 8; ++b) {     // branch-free: clamped index
        tmp[b] = src[min(base + b * PREP_THREADS + tid, n4 - 1)];
      }
#pragma unroll
      for (int b = 0; b < 8; ++b)       // duplicate stores at the clamp rewrite one value
        reinterpret_cast<float4 *>(stage)[min(base + b * PREP_THREADS + tid, n4 - 1)] = tmp[b];
    }
    __syncthreads();
    if (tid < cols) {
#pragma unroll 8
      for (int j = 0; j < nr; ++j) {
        const float m = stage[j * cols + tid];
        acc[0] = fmaf(m, qv[0][j0 + j], acc[0]);
        acc[1] = fmaf(m, qv[1][j0 + j], acc[1]);
        acc[2] = fmaf(m, qv[2][j0 + j], acc[2]);
        acc[3] = fmaf(m, qv[3][j0 + j], acc[3]);
      }
    }
  }
  if (tid < cols) {
    out[0][tid] = acc[0];
    out[1][tid] = acc[1];
    out[2][tid] = acc[2];
    out[3][tid] = acc[3];
  }
}

// out[hh][i] = sum_j MT[j][i] * qv[hh][j] with MT (row-major [d][cols]) already in LDS
__device__ inline void project_lds(const float *MT, int d, int cols, const float (*qv)[TQ_MAX_D],
                                   float (*out)[TQ_MAX_D]) {
  const int tid = threadIdx.x;
  if (tid < cols) {
    float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
#pragma unroll 8
    for (int j = 0; j < d; ++j) {
      const float m = MT[j * cols + tid];
      acc0 = fmaf(m, qv[0][j], acc0);
      acc1 = fmaf(m, qv[1][j], acc1);
      acc2 = fmaf(m, qv[2][j], acc2);
      acc3 = fmaf(m, qv[3][j], acc3);
    }
    out[0][tid] = acc0; out[1][tid] = acc1; out[2][tid] = acc2; out[3][tid] = acc3;
  }
}

#ifndef TQ_PREP_WAVES_PER_EU
#define TQ_PREP_WAVES_PER_EU 0
#endif
#if TQ_PREP_WAVES_PER_EU
__global__ void __launch_bounds__(PREP_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1))) prep_kernel(PrepArgs a) {
#else
__global__ void __launch_bounds__(PREP_THREADS) prep_kernel(PrepArgs a) {
#endif
  __shared__ float qv[4][TQ_MAX_D];
  __shared__ float qr[4][TQ_MAX_D];
  __shared__ float qs[4][TQ_MAX_D];
  __shared__ float vP[4][2 * 96 * 8];     // code-bit + parity-bit coefficients
  __shared__ float vQ[4][32 * 8];         // sign-bit coefficients
  __shared__ __align__(16) float stage[2 * PREP_STAGE_FLOATS];
  __shared__ float red[PREP_THREADS / 64][16];
  __shared__ float scal[4][2];
  __shared__ float sums[4][2];
  __shared__ float basis[4];

  const int gidx = blockIdx.x;           // = group * hg + head group
  const int grp = gidx / a.hg, hgi = gidx - grp * a.hg;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int d = a.d, m = a.m;
  const int ncb = a.cb * 8, nsb = a.sb * 8;
  // Kernel-argument fields are copied to LDS / scalars once: indexing them
  // with a runtime value makes the compiler re-load them from the kernarg
  // segment (a full memory round trip) on every use.
  if (tid < 4) basis[tid] = tid == 0 ? a.basis[0] : tid == 1 ? a.basis[1] : tid == 2 ? a.basis[2] : a.basis[3];
  const int w = a.w, cwpl = a.cb / 16, swpl = a.sb / 16;

  for (int i = tid; i < 4 * d; i += PREP_THREADS) {
    const int hh = i / d, j = i - hh * d;
    const int h = hgi * 4 + hh;
    const int64_t flat = (int64_t)grp * a.qpg + h;
    qv[hh][j] = (h < a.qpg && flat < a.nq_total) ? a.q[flat * d + j] : 0.f;
  }
  if (d <= 128) {
    // Pi^T and S^T (64 KB each at d = 128) fetched in one batch of 16-byte
    // loads per thread, then projected from LDS: one memory round trip.
    constexpr int B4 = 2 * PREP_STAGE_FLOATS / 4 / PREP_THREADS;     // float4s per thread per matrix
    const int n4p = d * d / 4, n4s = d * m / 4;
    const float4 *sp = reinterpret_cast<const float4 *>(a.PiT);
    const float4 *ss = reinterpret_cast<const float4 *>(a.ST);
    float4 *st4 = reinterpret_cast<float4 *>(stage);
    // unconditional clamped loads and stores: no branch, so every load of the
    // batch is in flight before the first LDS store waits
#pragma unroll
    for (int b = 0; b < B4; ++b) {
      const int i = min(b * PREP_THREADS + tid, n4p - 1);
      st4[i] = sp[i];
    }
    __syncthreads();
    project_lds(stage, d, d, qv, qr);
    __syncthreads();
    if (m) {
#pragma unroll
      for (int b = 0; b < B4; ++b) {
        const int i = min(b * PREP_THREADS + tid, n4s - 1);
        st4[i] = ss[i];
      }
      __syncthreads();
      project_lds(stage, d, m, qv, qs);
    }
  } else {
    __syncthreads();
    apply_T(a.PiT, d, d, qv, qr, stage);
    apply_T(a.ST, d, m, qv, qs, stage);
  }
  __syncthreads();

  // per-head sums of q_rot and q_s (for the +-1 -> bit conversion), one pass
  {
    float v[8];
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      v[2 * hh] = 0.f;
      v[2 * hh + 1] = 0.f;
      for (int i = tid; i < d; i += PREP_THREADS) v[2 * hh] += qr[hh][i];
      for (int i = tid; i < m; i += PREP_THREADS) v[2 * hh + 1] += qs[hh][i];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float t = wave_sum(v[k]);
      if (lane == 0) red[wv][k] = t;
    }
    __syncthreads();
    if (tid < 8) {
      float t = 0.f;
      for (int i = 0; i < PREP_THREADS / 64; ++i) t += red[i][tid];
      sums[tid >> 1][tid & 1] = t;
    }
  }

  // coefficients of every bit position
  const int npar = w == 3 ? ncb : 0;
  for (int i = tid; i < 4 * (ncb + npar); i += PREP_THREADS) {
    const int hh = i / (ncb + npar), k = i - hh * (ncb + npar);
    float v = 0.f;
    if (k < ncb) {
      const int coord = k / w, plane = k - coord * w;
      if (coord < d) v = 2.f * basis[plane] * qr[hh][coord];
    } else {
      const int kk = k - ncb;
      if (kk % 3 == 0 && kk / 3 < d) v = 2.f * basis[3] * qr[hh][kk / 3];
    }
    vP[hh][k] = v;
  }
  for (int i = tid; i < 4 * nsb; i += PREP_THREADS) {
    const int hh = i / nsb, k = i - hh * nsb;
    vQ[hh][k] = k < m ? 2.f * qs[hh][k] : 0.f;
  }
  __syncthreads();

  // per (head, chain) maxima of |v| 2^-j -> digit scale 127 / max, one pass
  {
    float v[8];
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      float mp = 0.f, mq = 0.f;
      for (int k = tid; k < ncb + npar; k += PREP_THREADS) mp = fmaxf(mp, ldexpf(fabsf(vP[hh][k]), -(k & 7)));
      for (int k = tid; k < nsb; k += PREP_THREADS) mq = fmaxf(mq, ldexpf(fabsf(vQ[hh][k]), -(k & 7)));
      v[2 * hh] = mp;
      v[2 * hh + 1] = mq;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float t = wave_max(v[k]);
      if (lane == 0) red[wv][8 + k] = t;
    }
    __syncthreads();
    if (tid < 8) {
      float t = 0.f;
      for (int i = 0; i < PREP_THREADS / 64; ++i) t = fmaxf(t, red[i][8 + tid]);
      scal[tid >> 1][tid & 1] = t > 0.f ? 127.f / t : 1.f;
    }
    __syncthreads();
  }

  uint8_t *out = a.ws + (int64_t)gidx * prep_stride(a.nm);
  // A fragments: dword index = (mu * 64 + lane) * 4 + e
  const int ndw = a.nm * 64 * 4;
  const int nmc = 2 * cwpl, nmp = w == 3 ? nmc : 0;
  for (int i = tid; i < ndw; i += PREP_THREADS) {
    const int mu = i >> 8, lane = (i >> 2) & 63, e = i & 3;
    const int row = lane & 15, g = lane >> 4;
    const int hh = row >> 2, digit = row & 3;
    int chain, mloc, wpl;
    const float *vv;
    if (mu < nmc + nmp) {
      chain = 0;
      const bool par = mu >= nmc;
      mloc = par ? mu - nmc : mu;
      wpl = cwpl;
      vv = vP[hh] + (par ? ncb : 0);
    } else {
      chain = 1;
      mloc = mu - nmc - nmp;
      wpl = swpl;
      vv = vQ[hh];
    }
    const int pair = mloc >> 1, half = mloc & 1;
    const int word = g * wpl + pair;
    const int j = 4 * half + e;
    const float S = scal[hh][chain];
    uint32_t dw = 0u;
    for (int b = 0; b < 4; ++b) {
      const int bitpos = 32 * word + 8 * b + j;
      float u = ldexpf(vv[bitpos] * S, -j);
      if (j == 7) u = -u;                 // B byte value is -128 for bit 7
      // base-128 digits, all four computed and one selected (no per-lane loop)
      const float r0 = rintf(u);
      u = (u - r0) * 128.f;
      const float r1 = rintf(u);
      u = (u - r1) * 128.f;
      const float r2 = rintf(u);
      u = (u - r2) * 128.f;
      const float r3 = rintf(u);
      const int dig = (int)(digit == 0 ? r0 : digit == 1 ? r1 : digit == 2 ? r2 : r3);
      dw |= ((uint32_t)(uint8_t)(int8_t)dig) << (8 * b);
    }
    reinterpret_cast<uint32_t *>(out)[i] = dw;
  }
  // constants per head: invS_P, invS_Q, K_P, K_Q
  if (tid < 4) {
    const int hh = tid;
    const float bsum = basis[0] + (w >= 2 ? basis[1] : 0.f) + (w >= 3 ? basis[2] + basis[3] : 0.f);
    float *cst = reinterpret_cast<float *>(out + (int64_t)a.nm * 1024);
    cst[hh * 4 + 0] = 1.f / scal[hh][0];
    cst[hh * 4 + 1] = 1.f / scal[hh][1];
    cst[hh * 4 + 2] = bsum * sums[hh][0];
    cst[hh * 4 + 3] = sums[hh][1];
  }
}

struct ScoreArgs {
  const uint8_t *codes, *signs;
  const float *norms, *rnorms;
  float *logits;
  const uint8_t *ws;
  int64_t T, ldk;
  int qpg, hg, tiles_per_wave, cb, sb;
  float alpha;
};

template <int CB16, int SB16, int W>
__global__ void __launch_bounds__(256) scores_kernel(ScoreArgs a) {
  constexpr int NM = ScoreShape<CB16, SB16, W>::NM;
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const int wv = threadIdx.x >> 6;
  const int64_t gidx = blockIdx.y;       // key group * hg + head group
  const int64_t kg = gidx / a.hg;
  const int hgi = (int)(gidx - kg * a.hg);

  const uint8_t *prep = a.ws + gidx * prep_stride(NM);
  i32x4 A[NM];
#pragma unroll
  for (int mu = 0; mu < NM; ++mu) A[mu] = reinterpret_cast<const i32x4 *>(prep)[mu * 64 + lane];
  const float *cst = reinterpret_cast<const float *>(prep + NM * 1024) + grp * 4;
  const HeadConsts hc{cst[0], cst[1], cst[2], cst[3]};
  const int head = hgi * 4 + grp;
  const bool head_ok = head < a.qpg;
  float *lrow = a.logits + ((int64_t)kg * a.qpg + (head_ok ? head : 0)) * a.T;

  // Record strides are compile-time (code_bytes = 16 CB16, sign_bytes = 16 SB16)
  // and per-token offsets are 32-bit from per-group base pointers, which keeps
  // address arithmetic to a few shifts per load.
  const uint8_t *cbase = a.codes + (int64_t)kg * a.ldk * (CB16 * 16);
  const uint8_t *sbase = a.signs + (int64_t)kg * a.ldk * (SB16 * 16);
  const float *nbase = a.norms + (int64_t)kg * a.ldk;
  const float *rbase = a.rnorms + (int64_t)kg * a.ldk;
  const int T = (int)a.T;                  // T < 2^31 is checked on the host

  const int tile0 = (blockIdx.x * 4 + wv) * a.tiles_per_wave;
  int ntile = a.tiles_per_wave;
  const int last = (T + 63) / 64;
  if (tile0 + ntile > last) ntile = last - tile0;
  auto load_tile = [&](KeyWords<CB16, SB16, W> (&kw)[4], float (&nu)[4], float (&ga)[4], int t0) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int t = min(t0 + 16 * s + col, T - 1);
      load_key_words(kw[s], cbase + (uint32_t)t * (CB16 * 16), sbase + (uint32_t)t * (SB16 * 16), grp);
      nu[s] = nbase[t];
      ga[s] = rbase[t];
    }
  };
  auto score_tile = [&](const KeyWords<CB16, SB16, W> (&kw)[4], const float (&nu)[4], const float (&ga)[4],
                        int t0) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int t = t0 + 16 * s + col;
      float l = tile_logit<CB16, SB16, W>(A, kw[s], nu[s], ga[s], a.alpha, hc);
      // Materialise l here: otherwise the compiler sinks the norm loads into
      // the guarded store and waits on each of them in turn.
      __asm__ volatile("" : "+v"(l));
      if (head_ok && t < T) lrow[t] = l;
    }
  };
#if TQ_SCORES_PREFETCH
  // two named register sets: the next tile's words load while this one is scored
  KeyWords<CB16, SB16, W> k0[4], k1[4];
  float n0[4], g0[4], n1[4], g1[4];
  if (ntile > 0) load_tile(k0, n0, g0, tile0 * 64);
  for (int it = 0; it < ntile; it += 2) {
    if (it + 1 < ntile) load_tile(k1, n1, g1, (tile0 + it + 1) * 64);
    score_tile(k0, n0, g0, (tile0 + it) * 64);
    if (it + 1 >= ntile) break;
    if (it + 2 < ntile) load_tile(k0, n0, g0, (tile0 + it + 2) * 64);
    score_tile(k1, n1, g1, (tile0 + it + 1) * 64);
  }
#else
  for (int it = 0; it < ntile; ++it) {
    KeyWords<CB16, SB16, W> kw[4];
    float nu[4], ga[4];
    load_tile(kw, nu, ga, (tile0 + it) * 64);
    score_tile(kw, nu, ga, (tile0 + it) * 64);
  }
#endif
}

int dispatch(const ScoreArgs &a, dim3 grid, int cb16, int sb16, int w, hipStream_t s) {
#define TQ_CASE(C, S, W_)                                        \
  if (cb16 == C && sb16 == S && w == W_) {                       \
    scores_kernel<C, S, W_><<<grid, 256, 0, s>>>(a);             \
    return hip_status();                                         \
  }
  TQ_FOR_EACH_GEOMETRY(TQ_CASE)
#undef TQ_CASE
  return TQ_ENOTSUP;
}

}  // namespace

int launch_prep(const tq_ctx *ctx, const float *q, int64_t groups, int qpg, int hg, int64_t nq_total,
                uint8_t *ws, hipStream_t stream) {
  PrepArgs pa{};
  pa.q = q;
  pa.PiT = ctx->PiT32;
  pa.ST = ctx->ST32;
  pa.ws = ws;
  pa.nq_total = nq_total;
  pa.d = ctx->hp.d;
  pa.m = ctx->hp.m;
  pa.w = ctx->hp.w;
  pa.qpg = qpg;
  pa.hg = hg;
  pa.cb = ctx->code_bytes;
  pa.sb = ctx->sign_bytes;
  pa.nm = mfma_count(ctx->code_bytes / 16, ctx->sign_bytes / 16, ctx->hp.w);
  for (int i = 0; i < 4; ++i) pa.basis[i] = ctx->basis[i];
  if (groups > 0x7fffffff) return TQ_ENOTSUP;
  prep_kernel<<<dim3((unsigned)groups), PREP_THREADS, 0, stream>>>(pa);
  return hip_status();
}

size_t scores_ws_bytes(const tq_ctx *ctx, int64_t G, int qpg) {
  const int hg = (qpg + 3) / 4;
  const int nm = mfma_count(ctx->code_bytes / 16, ctx->sign_bytes / 16, ctx->hp.w);
  return (size_t)(G * hg * prep_stride(nm));
}

int launch_scores(const tq_ctx *ctx, const float *q, int64_t G, int qpg, int64_t T, int64_t ldk,
                  const uint8_t *codes, const uint8_t *signs, const float *norms,
                  const float *rnorms, float *logits, void *ws, hipStream_t stream) {
  if (G == 0 || T == 0) return TQ_OK;
  const int hg = (qpg + 3) / 4;
  const int cb16 = ctx->code_bytes / 16, sb16 = ctx->sign_bytes / 16, w = ctx->hp.w;
  const int64_t groups = G * hg;
  if (groups > 65535 || T > 0x7fffffff - 64) return TQ_ENOTSUP;
  int st = launch_prep(ctx, q, groups, qpg, hg, G * qpg, reinterpret_cast<uint8_t *>(ws), stream);
  if (st != TQ_OK) return st;

  ScoreArgs sa{};
  sa.codes = codes;
  sa.signs = signs;
  sa.norms = norms;
  sa.rnorms = rnorms;
  sa.logits = logits;
  sa.ws = reinterpret_cast<const uint8_t *>(ws);
  sa.T = T;
  sa.ldk = ldk;
  sa.qpg = qpg;
  sa.hg = hg;
  sa.cb = ctx->code_bytes;
  sa.sb = ctx->sign_bytes;
  sa.alpha = ctx->alpha;
  // key tiles of 64 per wave iteration; aim for ~TQ_SCORES_WAVES waves overall
  const int64_t tiles = (T + 63) / 64;
  int64_t tpw = (tiles * groups + TQ_SCORES_WAVES - 1) / TQ_SCORES_WAVES;
  if (tpw < 1) tpw = 1;
  if (tpw > 64) tpw = 64;
  const int64_t chunks = (tiles + 4 * tpw - 1) / (4 * tpw);
  sa.tiles_per_wave = (int)tpw;
  return dispatch(sa, dim3((unsigned)chunks, (unsigned)groups), cb16, sb16, w, stream);
}

// ------------------------------------------------------------------ softmax
// Row softmax of scale * logits.  A row of up to NT * 4 * VPT floats is held in
// registers (one HBM read, one write, 16-byte accesses); longer rows and rows
// whose length is not a multiple of 4 take a streaming two-pass kernel.
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// (max, sum-of-exp) pairs merged over the block: rows of 16 lanes by DPP
// (rescaling each partner's sum to the larger max), then through LDS.
__device__ inline void merge_ms(float &m, float &s, float m2, float s2) {
  const float mm = fmaxf(m, m2);
  s = (m == -INFINITY ? 0.f : s * exp2f((m - mm) * kLog2e)) + (m2 == -INFINITY ? 0.f : s2 * exp2f((m2 - mm) * kLog2e));
  m = mm;
}

template <int NT>
__device__ inline void block_max_sum(float &m, float &s) {
  __shared__ float sm[NT / 16], ss[NT / 16];
  merge_ms(m, s, dpp_f<0xb1>(m), dpp_f<0xb1>(s));
  merge_ms(m, s, dpp_f<0x4e>(m), dpp_f<0x4e>(s));
  merge_ms(m, s, dpp_f<0x141>(m), dpp_f<0x141>(s));
  merge_ms(m, s, dpp_f<0x140>(m), dpp_f<0x140>(s));
  if ((threadIdx.x & 15) == 0) {
    sm[threadIdx.x >> 4] = m;
    ss[threadIdx.x >> 4] = s;
  }
  __syncthreads();
  float M = sm[0];
  for (int i = 1; i < NT / 16; ++i) M = fmaxf(M, sm[i]);
  float S = 0.f;
  for (int i = 0; i < NT / 16; ++i) S += sm[i] == -INFINITY ? 0.f : ss[i] * exp2f((sm[i] - M) * kLog2e);
  m = M;
  s = S;
}

template <int NT, int VPT>
__global__ void __launch_bounds__(NT) softmax_reg_kernel(const float *in, float *out, int64_t T,
                                                          float scale) {
  const int64_t row = blockIdx.x;
  const float4 *x = reinterpret_cast<const float4 *>(in + row * T);
  float4 *y = reinterpret_cast<float4 *>(out + row * T);
  const int n4 = (int)(T >> 2);
  float4 v[VPT];
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int i = threadIdx.x + k * NT;
    if (i < n4) {
      v[k] = x[i];
      v[k].x *= scale; v[k].y *= scale; v[k].z *= scale; v[k].w *= scale;
      m = fmaxf(m, fmaxf(fmaxf(v[k].x, v[k].y), fmaxf(v[k].z, v[k].w)));
    }
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int i = threadIdx.x + k * NT;
    if (i < n4) {
      v[k].x = exp2f((v[k].x - m) * kLog2e);
      v[k].y = exp2f((v[k].y - m) * kLog2e);
      v[k].z = exp2f((v[k].z - m) * kLog2e);
      v[k].w = exp2f((v[k].w - m) * kLog2e);
      s += (v[k].x + v[k].y) + (v[k].z + v[k].w);
    }
  }
  const float mloc = m;
  block_max_sum<NT>(m, s);
  const float f = (mloc == -INFINITY ? 0.f : exp2f((mloc - m) * kLog2e)) / s;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int i = threadIdx.x + k * NT;
    if (i < n4) {
      float4 o = v[k];
      o.x *= f; o.y *= f; o.z *= f; o.w *= f;
      y[i] = o;
    }
  }
}

__global__ void __launch_bounds__(1024) softmax_stream_kernel(const float *in, float *out, int64_t T,
                                                              float scale) {
  const int64_t row = blockIdx.x;
  const float *x = in + row * T;
  float *y = out + row * T;
  float m = -INFINITY, s = 0.f;
  for (int64_t i = threadIdx.x; i < T; i += 1024) {
    const float z = scale * x[i];
    if (z > m) {
      s = (m == -INFINITY ? 0.f : s * exp2f((m - z) * kLog2e)) + 1.f;
      m = z;
    } else {
      s += exp2f((z - m) * kLog2e);
    }
  }
  block_max_sum<1024>(m, s);
  const float inv = 1.f / s;
  for (int64_t i = threadIdx.x; i < T; i += 1024) y[i] = exp2f((scale * x[i] - m) * kLog2e) * inv;
}

}  // namespace

int launch_softmax(const float *logits, int64_t rows, int64_t T, float scale, float *probs,
                   hipStream_t stream) {
  if (rows == 0 || T == 0) return TQ_OK;
  if (rows > 0x7fffffff) return TQ_ENOTSUP;
  const bool vec = (T % 4 == 0) && ((uintptr_t)logits % 16 == 0) && ((uintptr_t)probs % 16 == 0);
  const unsigned g = (unsigned)rows;
  if (vec && T <= 256 * 4 * 4) {
    softmax_reg_kernel<256, 4><<<g, 256, 0, stream>>>(logits, probs, T, scale);
  } else if (vec && T <= 256 * 4 * 32) {
    softmax_reg_kernel<256, 32><<<g, 256, 0, stream>>>(logits, probs, T, scale);
  } else if (vec && T <= 1024 * 4 * 16) {
    softmax_reg_kernel<1024, 16><<<g, 1024, 0, stream>>>(logits, probs, T, scale);
  } else {
    softmax_stream_kernel<<<g, 1024, 0, stream>>>(logits, probs, T, scale);
  }
  return hip_status();
}

}  // namespace tq
