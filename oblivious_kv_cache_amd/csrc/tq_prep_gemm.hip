// Query prep for many query groups at once (prefill-shaped calls: thousands
// of queries against one key set), d <= 256.  Two launches:
//
//  proj: the projections q_rot = Pi q and q_s = S q of the estimator
//    (hao.cnyes.com "TurboQuant", 1 bit 掃尾; suzuke blog, 第三步) as one GEMM
//    per block of 64 queries, Q [64 x d] times [Pi; S]^T [d x (d + m)], on
//    v_mfma_f32_16x16x32_bf16 with both operands split into three bf16 parts
//    (x = x_h + x_m + x_l, each part the bf16 rounding of what the previous
//    ones leave) and the six products of order <= 2 accumulated in fp32
//    (h h, h m, m h, m m, h l, l h): about 2^-26 relative error per product,
//    as fp32 FMA.  (A two-part split leaves ~2^-17, which moves logits near
//    zero by more than the estimator's 1e-4 absolute tolerance.)  Each wave
//    holds one 16-query tile of A in registers; the [Pi; S] fragments of one
//    16-column tile at a time are staged in LDS (double-buffered) and shared
//    by the four waves.  The projections of a group of 4 heads go to the
//    group's own workspace slot (nm KB >= 16 (d + m) bytes).
//  frag: one wave per group of 4 heads: the projections into LDS, per-head
//    sums and scaled maxima, then the int8 A fragments over the slot.  In a
//    quad of lanes (rows 4 head + digit of one lane group) lane t computes
//    the coefficients of byte t of its four dwords and all four base-128
//    digits of each; a byte transpose across the quad (DPP broadcasts) then
//    gives every lane its own digit of the four bytes.
#include "tq_quantize_body.h"
#include "tq_score_core.h"

namespace tq {
namespace {

struct PrepGemmArgs {
  const float *q;             // [G][qpg][d]
  uint8_t *ws;
  const Frag *MH, *MM, *ML;   // [Pi; S] fragments: row 16 u + r, column 32 k + 8 g + e
  int64_t nq_total, groups;
  int d, m, nk, ntile, w, qpg, hg, cb16, sb16, nm;
  float basis[4];
};

constexpr int PQB = 64;       // queries per projection block (16 groups of 4 heads)

template <int NK>
__global__ void __launch_bounds__(256) prep_proj_kernel(PrepGemmArgs a) {
  // B tile: [buffer][k-block][part h/m/l][64 lanes]
  __shared__ __align__(16) Frag bt[2][NK][3][64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r = lane & 15, g = lane >> 4;
  const int d = a.d, dm = a.d + a.m;
  const int64_t hg0 = (int64_t)blockIdx.x * (PQB / 4);
  // A: query row 16 wv + r of the block, k-group g
  const int lr = 16 * wv + r;
  const int64_t gidx = hg0 + lr / 4;
  const int hh = lr % 4;
  const int64_t grp = gidx / a.hg;
  const int h = (int)(gidx - grp * a.hg) * 4 + hh;
  const int64_t flat = grp * a.qpg + h;
  const bool live = gidx < a.groups && h < a.qpg && flat < a.nq_total;
  const float *qrow = a.q + (live ? flat : 0) * d;
  bf16x8 Ah[NK], Am[NK], Al[NK];
#pragma unroll
  for (int kb = 0; kb < NK; ++kb) {
    const int i0 = 32 * kb + 8 * g;                  // d % 8 == 0: a chunk is all in or all out
    float xs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) xs[e] = (live && i0 < d) ? qrow[i0 + e] : 0.f;   // q is 4-byte aligned
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      Ah[kb][e] = (__bf16)xs[e];
      const float r1 = xs[e] - (float)Ah[kb][e];     // exact in fp32
      Am[kb][e] = (__bf16)r1;
      Al[kb][e] = (__bf16)(r1 - (float)Am[kb][e]);
    }
  }
  // staging: thread tid moves fragments tid, tid + 256, ... of a tile; the
  // context holds nk = dpad / 32 <= NK k-blocks per tile, the others are zero
  constexpr int NF = NK * 3 * 64, PER = NF / 256;
  const int nk = a.nk;
  Frag pre[PER];
  auto fetch = [&](int u) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int f = tid + 256 * i, l = f & 63, part = (f >> 6) % 3, kb = (f >> 6) / 3;
      const Frag *src = part == 0 ? a.MH : part == 1 ? a.MM : a.ML;
      pre[i] = kb < nk ? src[(u * nk + kb) * 64 + l] : Frag{{0u, 0u, 0u, 0u}};
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PER; ++i) (&bt[buf][0][0][0])[tid + 256 * i] = pre[i];
  };
  // D rows 4 g + jj of query tile wv: group hg0 + 4 wv + g, head jj
  const int64_t gx = hg0 + 4 * wv + g;
  const bool sok = gx < a.groups;
  float *slot = reinterpret_cast<float *>(a.ws + (sok ? gx : 0) * prep_stride(a.nm));
  fetch(0);
  stash(0);
  __syncthreads();
  for (int u = 0; u < a.ntile; ++u) {
    const int buf = u & 1;
    if (u + 1 < a.ntile) fetch(u + 1);
    // two independent accumulation chains (small terms, large terms), added at the end
    f32x4 acs = f32x4{0.f, 0.f, 0.f, 0.f}, acl = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NK; ++kb) {
      const bf16x8 bh = as_bf(bt[buf][kb][0][lane]), bm = as_bf(bt[buf][kb][1][lane]),
                   bl = as_bf(bt[buf][kb][2][lane]);
      acs = mfma(Ah[kb], bl, acs);
      acl = mfma(Ah[kb], bm, acl);
      acs = mfma(Al[kb], bh, acs);
      acl = mfma(Am[kb], bh, acl);
      acs = mfma(Am[kb], bm, acs);
      acl = mfma(Ah[kb], bh, acl);
    }
    const int col = 16 * u + r;
    if (sok && col < dm) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) slot[jj * dm + col] = acl[jj] + acs[jj];
    }
    // the other buffer was last read before the previous barrier
    if (u + 1 < a.ntile) stash(buf ^ 1);
    __syncthreads();
  }
}

// The value of quad lane QP & 3 (DPP quad_perm broadcast).
template <int QP>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, QP, 0xf, 0xf, false);
}

__global__ void __launch_bounds__(256) prep_frag_kernel(PrepGemmArgs a) {
  __shared__ float prs[4][4 * 512];                 // per wave: 4 heads x (d + m) projections
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t gx = (int64_t)blockIdx.x * 4 + wv;
  if (gx >= a.groups) return;                       // no block-wide synchronisation below
  const int d = a.d, m = a.m, dm = d + m, w = a.w;
  float *pr = prs[wv];
  uint8_t *out = a.ws + gx * prep_stride(a.nm);
  const float *proj = reinterpret_cast<const float *>(out);
  for (int i = lane; i < 4 * dm; i += 64) pr[i] = proj[i];
  // orders the wave's LDS writes before its reads by other lanes, and its
  // reads of the slot before the slot is overwritten
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  wave_sync();
  float cb2[4];                                     // 2 basis[p]
#pragma unroll
  for (int p = 0; p < 4; ++p) cb2[p] = 2.f * a.basis[p];
  float sP[4] = {0.f, 0.f, 0.f, 0.f}, sQ[4] = {0.f, 0.f, 0.f, 0.f};
  float mP[4] = {0.f, 0.f, 0.f, 0.f}, mQ[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i = lane; i < d; i += 64) {
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      const float v = pr[hh * dm + i], av = fabsf(v);
      sP[hh] += v;
      for (int p = 0; p < w; ++p) mP[hh] = fmaxf(mP[hh], ldexpf(fabsf(cb2[p]) * av, -((i * w + p) & 7)));
      if (w == 3) mP[hh] = fmaxf(mP[hh], ldexpf(fabsf(cb2[3]) * av, -((3 * i) & 7)));
    }
  }
  for (int jj = lane; jj < m; jj += 64) {
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      const float v = pr[hh * dm + d + jj];
      sQ[hh] += v;
      mQ[hh] = fmaxf(mQ[hh], ldexpf(2.f * fabsf(v), -(jj & 7)));
    }
  }
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    sP[hh] = wave_sum(sP[hh]);
    sQ[hh] = wave_sum(sQ[hh]);
    mP[hh] = wave_max(mP[hh]);
    mQ[hh] = wave_max(mQ[hh]);
  }
  // lane: fragment row r = 4 head + t of lane group g; it computes the
  // coefficients of byte t of each of its dwords
  const int r = lane & 15, g = lane >> 4, hr = r >> 2, t = r & 3;
  const float mx0 = hr == 0 ? mP[0] : hr == 1 ? mP[1] : hr == 2 ? mP[2] : mP[3];
  const float mx1 = hr == 0 ? mQ[0] : hr == 1 ? mQ[1] : hr == 2 ? mQ[2] : mQ[3];
  const float sc0 = mx0 > 0.f ? 127.f / mx0 : 1.f, sc1 = mx1 > 0.f ? 127.f / mx1 : 1.f;
  const float *qr = pr + hr * dm, *qs = qr + d;
  const int cwpl = a.cb16, swpl = a.sb16;
  const int nmc = 2 * cwpl, nmp = 2 * parity_words(cwpl, w);
  // byte selector: byte t of the low operand, byte t of the high operand
  const uint32_t psel = (uint32_t)t | ((uint32_t)(4 + t) << 8) | 0x0c0c0000u;
  wave_sync();                                      // every lane has read the slot
  for (int mu = 0; mu < a.nm; ++mu) {
    int kind, mloc, wpl;         // kind 0: code bits, 1: merged parity bits, 2: sign bits
    if (mu < nmc) {
      kind = 0; mloc = mu; wpl = cwpl;
    } else if (mu < nmc + nmp) {
      kind = 1; mloc = mu - nmc; wpl = cwpl;
    } else {
      kind = 2; mloc = mu - nmc - nmp; wpl = swpl;
    }
    const float S = kind == 2 ? sc1 : sc0;
    const int pair = mloc >> 1, half = mloc & 1;
    uint32_t dig[4];                               // [e]: the four digits of byte t's coefficient
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = 4 * half + e, q = 8 * t + j;
      // merged parity word `pair`: bit q belongs to the code starting at bit
      // q of record word g*wpl + p, p = 3 pair + ((q - g*wpl) mod 3)
      const int p = kind == 1 ? 3 * pair + ((q - g * wpl) % 3 + 3) % 3 : pair;
      const int bitpos = 32 * (g * wpl + p) + q;
      float v = 0.f;
      if (p < wpl) {
        if (kind == 0) {
          // bitpos / w for w in {1, 2, 3} (the last exact below 2^15)
          const int i = w == 1 ? bitpos : w == 2 ? bitpos >> 1 : (bitpos * 43691) >> 17;
          const int pl = bitpos - i * w;
          if (i < d) v = (pl == 0 ? cb2[0] : pl == 1 ? cb2[1] : cb2[2]) * qr[i];
        } else if (kind == 1) {
          const int i = (bitpos * 43691) >> 17;
          if (bitpos - 3 * i == 0 && i < d) v = cb2[3] * qr[i];
        } else if (bitpos < m) {
          v = 2.f * qs[bitpos];
        }
      }
      // U = u 2^21 rounded, u = v S 2^-j (negated for j = 7: the B byte value
      // is -128), split into balanced base-128 digits U = r0 2^21 + r1 2^14 +
      // r2 2^7 + r3, |r1|, |r2| <= 64, r3 in [-64, 64)
      const int U = (int)rintf(ldexpf((e == 3 && half) ? -v * S : v * S, 21 - j));
      const int r0 = (U + (1 << 20)) >> 21;
      const int R1 = U - (r0 << 21);
      const int r1 = (R1 + (1 << 13)) >> 14;
      const int R2 = R1 - (r1 << 14);
      const int r2 = (R2 + 64) >> 7;
      const int r3 = R2 - (r2 << 7);
      dig[e] = (uint32_t)(r0 & 0xff) | ((uint32_t)(r1 & 0xff) << 8) | ((uint32_t)(r2 & 0xff) << 16) |
               ((uint32_t)r3 << 24);
    }
    // dword e of this lane: byte b = digit t of quad lane b's coefficient e
    // (v_perm_b32: bytes t of two dwords side by side, then the two pairs)
    uint32_t dw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t x0 = quad_bcast<0x00>(dig[e]), x1 = quad_bcast<0x55>(dig[e]);
      const uint32_t x2 = quad_bcast<0xaa>(dig[e]), x3 = quad_bcast<0xff>(dig[e]);
      const uint32_t p01 = __builtin_amdgcn_perm(x1, x0, psel), p23 = __builtin_amdgcn_perm(x3, x2, psel);
      dw[e] = __builtin_amdgcn_perm(p23, p01, 0x05040100u);
    }
    *reinterpret_cast<uint4 *>(out + ((int64_t)mu * 64 + lane) * 16) = make_uint4(dw[0], dw[1], dw[2], dw[3]);
  }
  if (lane < 4) {
    const float xp = lane == 0 ? mP[0] : lane == 1 ? mP[1] : lane == 2 ? mP[2] : mP[3];
    const float xq = lane == 0 ? mQ[0] : lane == 1 ? mQ[1] : lane == 2 ? mQ[2] : mQ[3];
    const float s0 = lane == 0 ? sP[0] : lane == 1 ? sP[1] : lane == 2 ? sP[2] : sP[3];
    const float s1 = lane == 0 ? sQ[0] : lane == 1 ? sQ[1] : lane == 2 ? sQ[2] : sQ[3];
    const float bsum = a.basis[0] + (w >= 2 ? a.basis[1] : 0.f) + (w >= 3 ? a.basis[2] + a.basis[3] : 0.f);
    float *cst = reinterpret_cast<float *>(out + (int64_t)a.nm * 1024);
    cst[lane * 4 + 0] = xp > 0.f ? 1.f / (127.f / xp) : 1.f;
    cst[lane * 4 + 1] = xq > 0.f ? 1.f / (127.f / xq) : 1.f;
    cst[lane * 4 + 2] = bsum * s0;
    cst[lane * 4 + 3] = s1;
  }
}

}  // namespace

bool prep_gemm_applies(const tq_ctx *ctx, int64_t groups) {
  return ctx->PqH != nullptr && groups >= 1024;
}

int launch_prep_gemm(const tq_ctx *ctx, const float *q, int64_t groups, int qpg, int hg, int64_t nq_total,
                     uint8_t *ws, hipStream_t stream) {
  PrepGemmArgs a{};
  a.q = q;
  a.ws = ws;
  a.MH = ctx->PqH;
  a.MM = ctx->PqH + ctx->npq;
  a.ML = ctx->PqH + 2 * ctx->npq;
  a.nq_total = nq_total;
  a.groups = groups;
  a.d = ctx->hp.d;
  a.m = ctx->hp.m;
  a.ntile = (a.d + a.m + 15) / 16;
  a.nk = ctx->dpad / 32;
  a.w = ctx->hp.w;
  a.qpg = qpg;
  a.hg = hg;
  a.cb16 = ctx->cw16;
  a.sb16 = ctx->sign_bytes / 16;
  a.nm = mfma_count(a.cb16, a.sb16, a.w);
  for (int i = 0; i < 4; ++i) a.basis[i] = ctx->basis[i];
  const int nk = a.nk;
  const int64_t pblocks = (groups + PQB / 4 - 1) / (PQB / 4), fblocks = (groups + 3) / 4;
  if (pblocks > 0x7fffffff || fblocks > 0x7fffffff || a.d + a.m > 512) return TQ_ENOTSUP;
  if (nk <= 4)
    prep_proj_kernel<4><<<(unsigned)pblocks, 256, 0, stream>>>(a);
  else if (nk <= 8)
    prep_proj_kernel<8><<<(unsigned)pblocks, 256, 0, stream>>>(a);
  else
    return TQ_ENOTSUP;
  if (hip_status() != TQ_OK) return TQ_EHIP;
  prep_frag_kernel<<<(unsigned)fblocks, 256, 0, stream>>>(a);
  return hip_status();
}

}  // namespace tq
