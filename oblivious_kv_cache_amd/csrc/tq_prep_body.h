// Query-prep body of the estimator (see tq_scores.hip for the math): the
// per-(KV group, 4-head block) int8 operand fragments and constants.
#pragma once

#include "tq_score_core.h"

namespace tq {
namespace {

constexpr int PREP_THREADS = 256;

struct PrepArgs {
  const float *q;      // [G][qpg][d]
  const float *PiT;    // [d][d]
  const float *ST;     // [d][m]
  uint8_t *ws;
  int64_t nq_total;    // queries beyond this flat index are zero
  int d, m, w, qpg, hg, cb, sb, nm;
  float basis[4];
  // fractional widths (planar quarters): code words per lane group, the
  // second half's code bits and odd-basis coefficients
  int frac, cw16, w2;
  float basis2[4];
};

// Shared memory of one query-prep group (about 48 KB at d <= 128)
template <bool SPLIT>
struct PrepSmem {
  __align__(16) float qT[256][4];             // queries, [coordinate][head]
  __align__(16) float part[SPLIT ? 2 * 4 * 128 * 4 : 4];   // [matrix][row group][column][head]
  float vP[4][2 * 96 * 8];                         // code-bit + parity-bit coefficients
  float vQ[4][32 * 8];                             // sign-bit coefficients
  float red[PREP_THREADS / 64][16];
};

// Build the int8 A fragments and per-head constants for one (group, head group).
//
// The kernel is latency-bound (one block per group, a few microseconds each),
// so it is laid out for few round trips and few barriers:
//   * d <= 128: threads [0, 128) project with Pi, [128, 256) with S, at once;
//     each loads a 4-column x JC/4-row block of Pi^T / S^T with one batch of
//     16-byte loads issued before the queries arrive, and the column's owner
//     adds the four row blocks' partial products;
//   * d > 128: one column per thread, both projections in turn, rows in
//     chunks of JC;
//   * the owner of a coordinate writes its bit coefficients and keeps the
//     partial sums and scaled maxima; one DPP + LDS reduction serves both;
//   * the fragments are written after the last barrier.
template <int JC, bool SPLIT>
__device__ __forceinline__ void prep_body(const PrepArgs &a, PrepSmem<SPLIT> &sm, int gidx, int tid,
                                          bool live) {
  float (&qT)[256][4] = sm.qT;
  float *part = sm.part;
  float (&vP)[4][2 * 96 * 8] = sm.vP;
  float (&vQ)[4][32 * 8] = sm.vQ;
  float (&red)[PREP_THREADS / 64][16] = sm.red;

  // gidx = group * hg + head group
  const int grp = gidx / a.hg, hgi = gidx - grp * a.hg;
  const int lane = tid & 63, wv = tid >> 6;
  const int d = a.d, m = a.m, w = a.w;
  // coefficient slots: record bit order, or for fractional widths the bits
  // of each lane group's word slots (32 (g cw16 + p) + q) then one parity
  // word per plane word of the first-half quarters
  const int cwpl = a.frac ? a.cw16 : a.cb / 16, swpl = a.sb / 16;
  const int wpp = d / 128;
  const int ncb = a.frac ? 4 * cwpl * 32 : a.cb * 8, nsb = a.sb * 8;
  const int npar = w == 3 ? (a.frac ? 4 * wpp * 32 : ncb) : 0;

  // d <= 128: thread (matrix, column quad, row group) loads RPG rows x 4
  // columns of Pi^T or S^T with 16-byte loads, issued before the queries
  // arrive (RPG <= 32 loads in flight per thread)
  constexpr int RPG = JC / 4;
  const int mat0 = SPLIT ? (tid >> 7) : 0;
  const int col = SPLIT ? (tid & 127) : tid;
  const int quad = col & 31, rg = col >> 5;
  float4 mq[SPLIT ? RPG : 1];
  if constexpr (SPLIT) {
    const float *MT = mat0 ? a.ST : a.PiT;
    const int cols = mat0 ? m : d;
    const int qc = min(quad, max(cols / 4, 1) - 1);
    if (cols > 0) {
#pragma unroll
      for (int jj = 0; jj < RPG; ++jj)
        mq[jj] = *reinterpret_cast<const float4 *>(MT + min(rg * RPG + jj, d - 1) * cols + 4 * qc);
    }
  }

  // queries (rows past d are zero, so clamped matrix rows add nothing)
  const int nrow = SPLIT ? JC : d;
  for (int i = tid; i < 4 * nrow; i += PREP_THREADS) {
    const int hh = i / nrow, j = i - hh * nrow;
    const int h = hgi * 4 + hh;
    const int64_t flat = (int64_t)grp * a.qpg + h;
    qT[j][hh] = (j < d && h < a.qpg && flat < a.nq_total) ? a.q[flat * d + j] : 0.f;
  }
  for (int i = tid; i < 4 * (ncb + npar); i += PREP_THREADS) (&vP[0][0])[(i / (ncb + npar)) * (2 * 96 * 8) + i % (ncb + npar)] = 0.f;
  for (int i = tid; i < 4 * nsb; i += PREP_THREADS) (&vQ[0][0])[(i / nsb) * (32 * 8) + i % nsb] = 0.f;
  __syncthreads();

  float accS[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (SPLIT) {
    // partial products of this thread's rows, then the 4 row groups summed
    // by the column's owner
    float pc[4][4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) pc[c][hh] = 0.f;
#pragma unroll
    for (int jj = 0; jj < RPG; ++jj) {
      const float4 q4 = *reinterpret_cast<const float4 *>(&qT[rg * RPG + jj][0]);
      const float mv[4] = {mq[jj].x, mq[jj].y, mq[jj].z, mq[jj].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        pc[c][0] = fmaf(mv[c], q4.x, pc[c][0]);
        pc[c][1] = fmaf(mv[c], q4.y, pc[c][1]);
        pc[c][2] = fmaf(mv[c], q4.z, pc[c][2]);
        pc[c][3] = fmaf(mv[c], q4.w, pc[c][3]);
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *reinterpret_cast<float4 *>(&part[(((mat0 * 4 + rg) * 128) + 4 * quad + c) * 4]) =
          make_float4(pc[c][0], pc[c][1], pc[c][2], pc[c][3]);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float4 v = *reinterpret_cast<const float4 *>(&part[(((mat0 * 4 + r) * 128) + col) * 4]);
      accS[0] += v.x;
      accS[1] += v.y;
      accS[2] += v.z;
      accS[3] += v.w;
    }
  }

  // per thread: sums (P: code chain, Q: sign chain) and maxima of |v| 2^-(bit & 7)
  float sP[4] = {0.f, 0.f, 0.f, 0.f}, sQ[4] = {0.f, 0.f, 0.f, 0.f};
  float mP[4] = {0.f, 0.f, 0.f, 0.f}, mQ[4] = {0.f, 0.f, 0.f, 0.f};
  for (int mat = mat0; mat < (SPLIT ? mat0 + 1 : 2); ++mat) {
    const int cols = mat ? m : d;
    float acc[4] = {accS[0], accS[1], accS[2], accS[3]};
    if constexpr (!SPLIT) {
      // d > 128: one column per thread, rows in chunks of JC
      const float *MT = mat ? a.ST : a.PiT;
      const int c = min(col, max(cols, 1) - 1);
      for (int j0 = 0; j0 < d; j0 += JC) {
        float mc[JC];
#pragma unroll
        for (int j = 0; j < JC; ++j) mc[j] = MT[min(j0 + j, d - 1) * cols + c];
#pragma unroll
        for (int j = 0; j < JC; ++j) {
          if (j0 + j < d) {
            const float4 q4 = *reinterpret_cast<const float4 *>(&qT[j0 + j][0]);
            acc[0] = fmaf(mc[j], q4.x, acc[0]);
            acc[1] = fmaf(mc[j], q4.y, acc[1]);
            acc[2] = fmaf(mc[j], q4.z, acc[2]);
            acc[3] = fmaf(mc[j], q4.w, acc[3]);
          }
        }
      }
    }
    if (col < cols && mat == 0 && a.frac) {
      // quarter g of coordinate col: plane pl of word slot pl wpp + jq / 32
      const int qd = d / 4, g4 = col / qd, jq = col - g4 * qd;
      const bool second = g4 >= 2;
      const int cw = second ? a.w2 : w;
      const float *bs = second ? a.basis2 : a.basis;
      const float bsum = bs[0] + (cw >= 2 ? bs[1] : 0.f) + (cw >= 3 ? bs[2] + bs[3] : 0.f);
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        sP[hh] = bsum * acc[hh];
        for (int pl = 0; pl < cw; ++pl) {
          const int pos = 32 * (g4 * cwpl + pl * wpp + (jq >> 5)) + (jq & 31);
          const float v = 2.f * bs[pl] * acc[hh];
          vP[hh][pos] = v;
          mP[hh] = fmaxf(mP[hh], ldexpf(fabsf(v), -(jq & 7)));
        }
        if (cw == 3) {
          const int pos = 32 * (g4 * wpp + (jq >> 5)) + (jq & 31);
          const float v = 2.f * bs[3] * acc[hh];
          vP[hh][ncb + pos] = v;
          mP[hh] = fmaxf(mP[hh], ldexpf(fabsf(v), -(jq & 7)));
        }
      }
    } else if (col < cols) {
      if (mat == 0) {
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) {
          sP[hh] = acc[hh];
#pragma unroll
          for (int p = 0; p < 3; ++p) {
            if (p < w) {
              const int pos = col * w + p;
              const float v = 2.f * a.basis[p] * acc[hh];
              vP[hh][pos] = v;
              mP[hh] = fmaxf(mP[hh], ldexpf(fabsf(v), -(pos & 7)));
            }
          }
          if (w == 3) {
            const int pos = 3 * col;
            const float v = 2.f * a.basis[3] * acc[hh];
            vP[hh][ncb + pos] = v;
            mP[hh] = fmaxf(mP[hh], ldexpf(fabsf(v), -(pos & 7)));
          }
        }
      } else {
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) {
          sQ[hh] = acc[hh];
          const float v = 2.f * acc[hh];
          vQ[hh][col] = v;
          mQ[hh] = ldexpf(fabsf(v), -(col & 7));
        }
      }
    }
  }
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    const float t0 = wave_sum(sP[hh]), t1 = wave_sum(sQ[hh]);
    const float t2 = wave_max(mP[hh]), t3 = wave_max(mQ[hh]);
    if (lane == 0) {
      red[wv][2 * hh] = t0;
      red[wv][2 * hh + 1] = t1;
      red[wv][8 + 2 * hh] = t2;
      red[wv][8 + 2 * hh + 1] = t3;
    }
  }
  __syncthreads();

  uint8_t *out = a.ws + (int64_t)gidx * prep_stride(a.nm);
  // A fragments: dword index i = (mu * 64 + lane) * 4 + e; thread tid writes
  // dword tid of every mu, so its lane (row -> head, digit) and e are fixed
  const int flane = tid >> 2, e = tid & 3;
  const int row = flane & 15, g = flane >> 4;
  const int hh = row >> 2, digit = row & 3;
  float mx0 = 0.f, mx1 = 0.f;
#pragma unroll
  for (int i = 0; i < PREP_THREADS / 64; ++i) {
    mx0 = fmaxf(mx0, red[i][8 + 2 * hh]);
    mx1 = fmaxf(mx1, red[i][8 + 2 * hh + 1]);
  }
  const float sc0 = mx0 > 0.f ? 127.f / mx0 : 1.f, sc1 = mx1 > 0.f ? 127.f / mx1 : 1.f;
  const int nmc = 2 * cwpl, nmp = 2 * parity_words(cwpl, w);
  for (int mu = 0; mu < a.nm; ++mu) {
    int mloc, wpl;
    const float *vv;
    float S;
    bool par = false;
    if (mu < nmc + nmp) {
      par = mu >= nmc;
      mloc = par ? mu - nmc : mu;
      wpl = cwpl;
      vv = vP[hh] + (par ? ncb : 0);
      S = sc0;
    } else {
      mloc = mu - nmc - nmp;
      wpl = swpl;
      vv = vQ[hh];
      S = sc1;
    }
    const int pair = mloc >> 1, half = mloc & 1;
    const int j = 4 * half + e;
    uint32_t dw = 0u;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int q = 8 * b + j;
      // merged parity word `pair`: bit q belongs to the code starting at bit
      // q of record word g*wpl + p, p = 3 pair + ((q - g*wpl) mod 3), if any
      // (fractional widths: parity word `pair` is plane word `pair`, unmerged)
      const int p = par && !a.frac ? 3 * pair + ((q - g * wpl) % 3 + 3) % 3 : pair;
      const int pw = par && a.frac ? wpp : wpl;
      const int bitpos = 32 * (g * pw + p) + q;
      float u = p < pw ? ldexpf(vv[bitpos] * S, -j) : 0.f;
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
    if (live) reinterpret_cast<uint32_t *>(out)[mu * 256 + tid] = dw;
  }
  // constants per head: invS_P, invS_Q, K_P, K_Q
  if (live && tid < 4) {
    const int h4 = tid;
    float s0 = 0.f, s1 = 0.f, x0 = 0.f, x1 = 0.f;
#pragma unroll
    for (int i = 0; i < PREP_THREADS / 64; ++i) {
      s0 += red[i][2 * h4];
      s1 += red[i][2 * h4 + 1];
      x0 = fmaxf(x0, red[i][8 + 2 * h4]);
      x1 = fmaxf(x1, red[i][8 + 2 * h4 + 1]);
    }
    const float bsum = a.basis[0] + (w >= 2 ? a.basis[1] : 0.f) + (w >= 3 ? a.basis[2] + a.basis[3] : 0.f);
    float *cst = reinterpret_cast<float *>(out + (int64_t)a.nm * 1024);
    cst[h4 * 4 + 0] = x0 > 0.f ? 1.f / (127.f / x0) : 1.f;
    cst[h4 * 4 + 1] = x1 > 0.f ? 1.f / (127.f / x1) : 1.f;
    cst[h4 * 4 + 2] = a.frac ? s0 : bsum * s0;      // fractional widths: s0 is already weighted
    cst[h4 * 4 + 3] = s1;
  }
}

// Kernel arguments of one query-prep job (groups of 4 heads: see launch_prep).
inline PrepArgs make_prep_args(const tq_ctx *ctx, const float *q, int qpg, int hg, int64_t nq_total,
                               uint8_t *ws) {
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
  pa.nm = mfma_count(ctx->cw16, ctx->sign_bytes / 16, ctx->hp.w);
  for (int i = 0; i < 4; ++i) {
    pa.basis[i] = ctx->basis[i];
    pa.basis2[i] = ctx->basis2[i];
  }
  pa.frac = ctx->frac;
  pa.cw16 = ctx->cw16;
  pa.w2 = ctx->hp.w2;
  return pa;
}

}  // namespace
}  // namespace tq
