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
#include "tq_internal.h"

namespace tq {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int PREP_THREADS = 256;

struct ScoreGeom {
  int CB16, SB16, w, nm;   // code words/lane, sign words/lane, code bits, MFMAs per key tile
};

__host__ __device__ inline int mfma_count(int cb16, int sb16, int w) {
  return 2 * cb16 + (w == 3 ? 2 * cb16 : 0) + 2 * sb16;
}

// bytes of prepared query state per (KV group, head group)
__host__ __device__ inline int64_t prep_stride(int nm) {
  return ((int64_t)nm * 1024 + 64 + 255) / 256 * 256;
}

struct PrepArgs {
  const float *q;      // [G][qpg][d]
  const float *PiT;    // [d][d]
  const float *ST;     // [d][m]
  uint8_t *ws;
  int d, m, w, qpg, hg, cb, sb, nm;
  float basis[4];
};

// Build the int8 A fragments and per-head constants for one (group, head group).
__global__ void __launch_bounds__(PREP_THREADS) prep_kernel(PrepArgs a) {
  __shared__ float qv[4][TQ_MAX_D];
  __shared__ float qr[4][TQ_MAX_D];
  __shared__ float qs[4][TQ_MAX_D];
  __shared__ float vP[4][2 * 96 * 8];     // code-bit + parity-bit coefficients
  __shared__ float vQ[4][32 * 8];         // sign-bit coefficients
  __shared__ float red[4][2][PREP_THREADS / 64];
  __shared__ float scal[4][2];

  const int gidx = blockIdx.x;           // = group * hg + head group
  const int grp = gidx / a.hg, hgi = gidx - grp * a.hg;
  const int tid = threadIdx.x;
  const int d = a.d, m = a.m;
  const int ncb = a.cb * 8, nsb = a.sb * 8;

  for (int i = tid; i < 4 * d; i += PREP_THREADS) {
    const int hh = i / d, j = i - hh * d;
    const int h = hgi * 4 + hh;
    qv[hh][j] = h < a.qpg ? a.q[((int64_t)grp * a.qpg + h) * d + j] : 0.f;
  }
  __syncthreads();
  // q_rot = Pi q, q_s = S q  (PiT[j][i] = Pi[i][j]; ST[j][i] = S[i][j])
  if (tid < d) {
    float r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f;
    for (int j = 0; j < d; ++j) {
      const float p = a.PiT[(int64_t)j * d + tid];
      r0 = fmaf(p, qv[0][j], r0);
      r1 = fmaf(p, qv[1][j], r1);
      r2 = fmaf(p, qv[2][j], r2);
      r3 = fmaf(p, qv[3][j], r3);
    }
    qr[0][tid] = r0; qr[1][tid] = r1; qr[2][tid] = r2; qr[3][tid] = r3;
  }
  if (tid < m) {
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    for (int j = 0; j < d; ++j) {
      const float p = a.ST[(int64_t)j * m + tid];
      s0 = fmaf(p, qv[0][j], s0);
      s1 = fmaf(p, qv[1][j], s1);
      s2 = fmaf(p, qv[2][j], s2);
      s3 = fmaf(p, qv[3][j], s3);
    }
    qs[0][tid] = s0; qs[1][tid] = s1; qs[2][tid] = s2; qs[3][tid] = s3;
  }
  __syncthreads();

  // coefficients of every bit position
  const int npar = a.w == 3 ? ncb : 0;
  for (int i = tid; i < 4 * (ncb + npar); i += PREP_THREADS) {
    const int hh = i / (ncb + npar), k = i - hh * (ncb + npar);
    float v = 0.f;
    if (k < ncb) {
      const int coord = k / a.w, plane = k - coord * a.w;
      if (coord < d) v = 2.f * a.basis[plane] * qr[hh][coord];
    } else {
      const int kk = k - ncb;
      if (kk % 3 == 0 && kk / 3 < d) v = 2.f * a.basis[3] * qr[hh][kk / 3];
    }
    vP[hh][k] = v;
  }
  for (int i = tid; i < 4 * nsb; i += PREP_THREADS) {
    const int hh = i / nsb, k = i - hh * nsb;
    vQ[hh][k] = k < m ? 2.f * qs[hh][k] : 0.f;
  }
  __syncthreads();

  // per (head, chain) maxima of |v| 2^-j
  float mx[4][2];
  for (int hh = 0; hh < 4; ++hh) {
    float mp = 0.f, mq = 0.f;
    for (int k = tid; k < ncb + npar; k += PREP_THREADS) mp = fmaxf(mp, ldexpf(fabsf(vP[hh][k]), -(k & 7)));
    for (int k = tid; k < nsb; k += PREP_THREADS) mq = fmaxf(mq, ldexpf(fabsf(vQ[hh][k]), -(k & 7)));
    for (int o = 32; o > 0; o >>= 1) {
      mp = fmaxf(mp, __shfl_xor(mp, o));
      mq = fmaxf(mq, __shfl_xor(mq, o));
    }
    mx[hh][0] = mp;
    mx[hh][1] = mq;
  }
  if ((tid & 63) == 0)
    for (int hh = 0; hh < 4; ++hh) {
      red[hh][0][tid >> 6] = mx[hh][0];
      red[hh][1][tid >> 6] = mx[hh][1];
    }
  __syncthreads();
  if (tid < 8) {
    const int hh = tid >> 1, ch = tid & 1;
    float v = 0.f;
    for (int i = 0; i < PREP_THREADS / 64; ++i) v = fmaxf(v, red[hh][ch][i]);
    scal[hh][ch] = v > 0.f ? 127.f / v : 1.f;
  }
  __syncthreads();

  uint8_t *out = a.ws + (int64_t)gidx * prep_stride(a.nm);
  // A fragments: dword index = (mu * 64 + lane) * 4 + e
  const int ndw = a.nm * 64 * 4;
  const int nmc = 2 * (a.cb / 16), nmp = a.w == 3 ? nmc : 0;
  for (int i = tid; i < ndw; i += PREP_THREADS) {
    const int mu = i >> 8, lane = (i >> 2) & 63, e = i & 3;
    const int row = lane & 15, g = lane >> 4;
    const int hh = row >> 2, digit = row & 3;
    int chain, mloc, wpl, base;
    const float *vv;
    if (mu < nmc + nmp) {
      chain = 0;
      const bool par = mu >= nmc;
      mloc = par ? mu - nmc : mu;
      wpl = a.cb / 16;
      vv = vP[hh] + (par ? ncb : 0);
      base = 0;
    } else {
      chain = 1;
      mloc = mu - nmc - nmp;
      wpl = a.sb / 16;
      vv = vQ[hh];
      base = 0;
    }
    (void)base;
    const int pair = mloc >> 1, half = mloc & 1;
    const int word = g * wpl + pair;
    const int j = 4 * half + e;
    const float S = scal[hh][chain];
    uint32_t dw = 0u;
    for (int b = 0; b < 4; ++b) {
      const int bitpos = 32 * word + 8 * b + j;
      float u = ldexpf(vv[bitpos] * S, -j);
      if (j == 7) u = -u;                 // B byte value is -128 for bit 7
      int dig = 0;
      for (int t = 0; t <= digit; ++t) {
        const float r = rintf(u);
        dig = (int)r;
        u = (u - r) * 128.f;
      }
      dw |= ((uint32_t)(uint8_t)(int8_t)dig) << (8 * b);
    }
    reinterpret_cast<uint32_t *>(out)[i] = dw;
  }
  // constants per head: invS_P, invS_Q, K_P, K_Q
  if (tid < 4) {
    const int hh = tid;
    float sq = 0.f, ss = 0.f;
    for (int i = 0; i < d; ++i) sq += qr[hh][i];
    for (int i = 0; i < m; ++i) ss += qs[hh][i];
    float bsum = a.basis[0] + (a.w >= 2 ? a.basis[1] : 0.f) + (a.w >= 3 ? a.basis[2] + a.basis[3] : 0.f);
    float *cst = reinterpret_cast<float *>(out + (int64_t)a.nm * 1024);
    cst[hh * 4 + 0] = 1.f / scal[hh][0];
    cst[hh * 4 + 1] = 1.f / scal[hh][1];
    cst[hh * 4 + 2] = bsum * sq;
    cst[hh * 4 + 3] = ss;
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

__device__ __forceinline__ i32x4 mfma8(const i32x4 &a, const i32x4 &b, const i32x4 &c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ i32x4 planes(uint32_t w, int half) {
  const int s = 4 * half;
  return i32x4{(int)(w & (0x01010101u << s)), (int)(w & (0x01010101u << (s + 1))),
               (int)(w & (0x01010101u << (s + 2))), (int)(w & (0x01010101u << (s + 3)))};
}

template <int CB16, int SB16, int W>
__global__ void __launch_bounds__(256) scores_kernel(ScoreArgs a) {
  constexpr int NMC = 2 * CB16, NMP = (W == 3) ? 2 * CB16 : 0, NMS = 2 * SB16;
  constexpr int NM = NMC + NMP + NMS;
  constexpr int XW = (W == 3) ? 1 : 0;   // extra word for parity straddling
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
  const float invSP = cst[0], invSQ = cst[1], KP = cst[2], KQ = cst[3];
  const int head = hgi * 4 + grp;
  const bool head_ok = head < a.qpg;
  float *lrow = a.logits + ((int64_t)kg * a.qpg + head) * a.T;

  const uint8_t *cbase = a.codes + (int64_t)kg * a.ldk * a.cb + grp * (CB16 * 4);
  const uint8_t *sbase = a.signs + (int64_t)kg * a.ldk * a.sb + grp * (SB16 * 4);
  const float *nbase = a.norms + (int64_t)kg * a.ldk;
  const float *rbase = a.rnorms + (int64_t)kg * a.ldk;

  const int64_t tile0 = ((int64_t)blockIdx.x * 4 + wv) * a.tiles_per_wave;
  for (int it = 0; it < a.tiles_per_wave; ++it) {
    const int64_t t0 = (tile0 + it) * 64;
    if (t0 >= a.T) break;
    uint32_t cw[4][CB16 + XW], sw[4][SB16];
    float nu[4], ga[4];
    int64_t tk[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      int64_t t = t0 + 16 * s + col;
      tk[s] = t;
      if (t >= a.T) t = a.T - 1;
      const uint32_t *cp = reinterpret_cast<const uint32_t *>(cbase + t * a.cb);
#pragma unroll
      for (int i = 0; i < CB16; ++i) cw[s][i] = cp[i];
      if constexpr (XW) cw[s][CB16] = grp < 3 ? cp[CB16] : 0u;
      const uint32_t *sp = reinterpret_cast<const uint32_t *>(sbase + t * a.sb);
#pragma unroll
      for (int i = 0; i < SB16; ++i) sw[s][i] = sp[i];
      nu[s] = nbase[t];
      ga[s] = rbase[t];
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      i32x4 accP = {0, 0, 0, 0}, accQ = {0, 0, 0, 0};
#pragma unroll
      for (int p = 0; p < CB16; ++p) {
        accP = mfma8(A[2 * p], planes(cw[s][p], 0), accP);
        accP = mfma8(A[2 * p + 1], planes(cw[s][p], 1), accP);
      }
      if constexpr (W == 3) {
#pragma unroll
        for (int p = 0; p < CB16; ++p) {
          const uint32_t lo = cw[s][p], hi = cw[s][p + 1];
          const uint32_t par = lo ^ __builtin_amdgcn_alignbit(hi, lo, 1) ^ __builtin_amdgcn_alignbit(hi, lo, 2);
          accP = mfma8(A[NMC + 2 * p], planes(par, 0), accP);
          accP = mfma8(A[NMC + 2 * p + 1], planes(par, 1), accP);
        }
      }
#pragma unroll
      for (int p = 0; p < SB16; ++p) {
        accQ = mfma8(A[NMC + NMP + 2 * p], planes(sw[s][p], 0), accQ);
        accQ = mfma8(A[NMC + NMP + 2 * p + 1], planes(sw[s][p], 1), accQ);
      }
      const float P = fmaf((float)accP[3], 0x1.0p-21f,
                           fmaf((float)accP[2], 0x1.0p-14f, fmaf((float)accP[1], 0x1.0p-7f, (float)accP[0]))) *
                          invSP - KP;
      const float Q = fmaf((float)accQ[3], 0x1.0p-21f,
                           fmaf((float)accQ[2], 0x1.0p-14f, fmaf((float)accQ[1], 0x1.0p-7f, (float)accQ[0]))) *
                          invSQ - KQ;
      const float l = nu[s] * fmaf(a.alpha * ga[s], Q, P);
      if (head_ok && tk[s] < a.T) lrow[tk[s]] = l;
    }
  }
}

template <int CB16, int SB16, int W>
void launch_one(const ScoreArgs &a, dim3 grid, hipStream_t s) {
  scores_kernel<CB16, SB16, W><<<grid, 256, 0, s>>>(a);
}

int dispatch(const ScoreArgs &a, dim3 grid, int cb16, int sb16, int w, hipStream_t s) {
#define TQ_CASE(C, S, W_)                                   \
  if (cb16 == C && sb16 == S && w == W_) {                  \
    launch_one<C, S, W_>(a, grid, s);                       \
    return hip_status();                                    \
  }
  TQ_CASE(1, 1, 1) TQ_CASE(2, 2, 1) TQ_CASE(1, 2, 1)
  TQ_CASE(1, 1, 2) TQ_CASE(2, 1, 2) TQ_CASE(3, 2, 2) TQ_CASE(4, 2, 2)
  TQ_CASE(1, 1, 3) TQ_CASE(2, 1, 3) TQ_CASE(3, 1, 3) TQ_CASE(4, 2, 3) TQ_CASE(5, 2, 3) TQ_CASE(6, 2, 3)
#undef TQ_CASE
  return TQ_ENOTSUP;
}

}  // namespace

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
  const int nm = mfma_count(cb16, sb16, w);

  PrepArgs pa{};
  pa.q = q;
  pa.PiT = ctx->PiT32;
  pa.ST = ctx->ST32;
  pa.ws = reinterpret_cast<uint8_t *>(ws);
  pa.d = ctx->hp.d;
  pa.m = ctx->hp.m;
  pa.w = w;
  pa.qpg = qpg;
  pa.hg = hg;
  pa.cb = ctx->code_bytes;
  pa.sb = ctx->sign_bytes;
  pa.nm = nm;
  for (int i = 0; i < 4; ++i) pa.basis[i] = ctx->basis[i];
  prep_kernel<<<dim3((unsigned)(G * hg)), PREP_THREADS, 0, stream>>>(pa);
  if (hip_status() != TQ_OK) return TQ_EHIP;

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
  // key tiles of 64 per wave iteration; aim for >= ~4096 waves in flight overall
  const int64_t tiles = (T + 63) / 64;
  const int64_t groups = G * hg;
  int64_t tpw = (tiles * groups + 16383) / 16384;
  if (tpw < 1) tpw = 1;
  if (tpw > 64) tpw = 64;
  const int64_t chunks = (tiles + 4 * tpw - 1) / (4 * tpw);
  sa.tiles_per_wave = (int)tpw;
  if (groups > 65535) return TQ_ENOTSUP;
  return dispatch(sa, dim3((unsigned)chunks, (unsigned)groups), cb16, sb16, w, stream);
}

// ------------------------------------------------------------------ softmax
namespace {

__global__ void __launch_bounds__(256) softmax_kernel(const float *in, float *out, int64_t T,
                                                      float scale) {
  __shared__ float sm[4], ssum[4];
  const int64_t row = blockIdx.x;
  const float *x = in + row * T;
  float *y = out + row * T;
  float m = -INFINITY, s = 0.f;
  for (int64_t i = threadIdx.x; i < T; i += 256) {
    const float z = scale * x[i];
    if (z > m) {
      s = s * expf(m - z) + 1.f;
      m = z;
    } else {
      s += expf(z - m);
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o);
    const float mm = fmaxf(m, m2);
    s = (m == -INFINITY ? 0.f : s * expf(m - mm)) + (m2 == -INFINITY ? 0.f : s2 * expf(m2 - mm));
    m = mm;
  }
  if ((threadIdx.x & 63) == 0) {
    sm[threadIdx.x >> 6] = m;
    ssum[threadIdx.x >> 6] = s;
  }
  __syncthreads();
  float M = sm[0];
  for (int i = 1; i < 4; ++i) M = fmaxf(M, sm[i]);
  float S = 0.f;
  for (int i = 0; i < 4; ++i) S += sm[i] == -INFINITY ? 0.f : ssum[i] * expf(sm[i] - M);
  const float inv = 1.f / S;
  for (int64_t i = threadIdx.x; i < T; i += 256) y[i] = expf(scale * x[i] - M) * inv;
}

}  // namespace

int launch_softmax(const float *logits, int64_t rows, int64_t T, float scale, float *probs,
                   hipStream_t stream) {
  if (rows == 0 || T == 0) return TQ_OK;
  if (rows > 0x7fffffff) return TQ_ENOTSUP;
  softmax_kernel<<<(unsigned)rows, 256, 0, stream>>>(logits, probs, T, scale);
  return hip_status();
}

}  // namespace tq
