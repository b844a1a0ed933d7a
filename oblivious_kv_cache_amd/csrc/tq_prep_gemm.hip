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
//    holds one 16-query tile of A in registers; the [Pi; S] fragments of
//    several 16-column tiles at a time are staged in LDS and shared by the
//    block's sixteen waves.  The projections of a group of 4 heads go to the
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
  int q16;                    // q on 16 bytes (then its rows are too: d % 8 == 0)
  float basis[4];
};

// waves (query tiles of 16) per projection block: 16, or 8 where the A
// fragments of d > 128 need more than 128 VGPRs
__host__ __device__ constexpr int proj_waves(int nk) { return nk > 4 ? 8 : 16; }

// The [Pi; S] fragments are the same for every block, so a block takes many
// queries (8 or 16 waves of 16) and stages the fragments of several
// 16-column tiles at once (96 KB of LDS per pass, one barrier per pass): the
// block's time is then its MFMAs and stores, not one L2 round trip per tile.
template <int NK>
__global__ void __launch_bounds__(64 * proj_waves(NK)) prep_proj_kernel(PrepGemmArgs a) {
  constexpr int NW = proj_waves(NK);
  constexpr int TP = 32 / NK;                        // column tiles per pass
  // B tiles of a pass: [tile][k-block][part h/m/l][64 lanes]
  __shared__ __align__(16) Frag bt[TP][NK][3][64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r = lane & 15, g = lane >> 4;
  const int d = a.d, dm = a.d + a.m;
  const int64_t hg0 = (int64_t)blockIdx.x * (4 * NW);
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
  // the lane's 8-coordinate chunks, all loads issued before any is used
  // (d % 8 == 0: a chunk is all in or all out; with q on 16 bytes every
  // chunk is, so it takes two 16-byte loads)
  float4 xv[NK][2];
#pragma unroll
  for (int kb = 0; kb < NK; ++kb) {
    const int i0 = 32 * kb + 8 * g;
    const bool in = live && i0 < d;
    const float *src = qrow + (in ? i0 : 0);
    if (a.q16) {
      xv[kb][0] = in ? reinterpret_cast<const float4 *>(src)[0] : make_float4(0.f, 0.f, 0.f, 0.f);
      xv[kb][1] = in ? reinterpret_cast<const float4 *>(src)[1] : make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
      xv[kb][0] = in ? make_float4(src[0], src[1], src[2], src[3]) : make_float4(0.f, 0.f, 0.f, 0.f);
      xv[kb][1] = in ? make_float4(src[4], src[5], src[6], src[7]) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
#pragma unroll
  for (int kb = 0; kb < NK; ++kb) {
    const float xs[8] = {xv[kb][0].x, xv[kb][0].y, xv[kb][0].z, xv[kb][0].w,
                         xv[kb][1].x, xv[kb][1].y, xv[kb][1].z, xv[kb][1].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      Ah[kb][e] = (__bf16)xs[e];
      const float r1 = xs[e] - (float)Ah[kb][e];     // exact in fp32
      Am[kb][e] = (__bf16)r1;
      Al[kb][e] = (__bf16)(r1 - (float)Am[kb][e]);
    }
  }
  // D rows 4 g + jj of query tile wv: group hg0 + 4 wv + g, head jj
  const int64_t gx = hg0 + 4 * wv + g;
  const bool sok = gx < a.groups;
  float *slot = reinterpret_cast<float *>(a.ws + (sok ? gx : 0) * prep_stride(a.nm));
  const int nk = a.nk;                               // the context's k-blocks (<= NK; the A beyond is zero)
  for (int u0 = 0; u0 < a.ntile; u0 += TP) {
    const int nt = min(TP, a.ntile - u0);
    if (u0 > 0) __syncthreads();                     // the previous pass's tiles are all read
    // the pass's fragments, 1 KB (one fragment of 64 lanes) per copy, copied
    // into LDS by the memory system; wave wv takes entries wv, wv + NW, ...
    constexpr int NE = TP * NK * 3;
#pragma unroll
    for (int i = 0; i < (NE + NW - 1) / NW; ++i) {
      const int e = wv + NW * i, ul = e / (3 * NK), kb = (e / 3) % NK, part = e % 3;
      if (e < NE && ul < nt && kb < nk) {
        const Frag *src = part == 0 ? a.MH : part == 1 ? a.MM : a.ML;
        __builtin_amdgcn_global_load_lds(src + ((u0 + ul) * nk + kb) * 64 + lane,
                                         (__attribute__((address_space(3))) void *)&bt[ul][kb][part][0], 16, 0, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);              // vmcnt(0): this wave's copies are in LDS
    __syncthreads();
    for (int ul = 0; ul < nt; ++ul) {
      // two independent accumulation chains (small terms, large terms), added at the end
      f32x4 acs = f32x4{0.f, 0.f, 0.f, 0.f}, acl = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NK; ++kb) {
        if (kb >= nk) break;                         // (only copied k-blocks are read)
        const bf16x8 bh = as_bf(bt[ul][kb][0][lane]), bm = as_bf(bt[ul][kb][1][lane]),
                     bl = as_bf(bt[ul][kb][2][lane]);
        acs = mfma(Ah[kb], bl, acs);
        acl = mfma(Ah[kb], bm, acl);
        acs = mfma(Al[kb], bh, acs);
        acl = mfma(Am[kb], bh, acl);
        acs = mfma(Am[kb], bm, acs);
        acl = mfma(Ah[kb], bh, acl);
      }
      const int col = 16 * (u0 + ul) + r;
      if (sok && col < dm)                           // [column][head]: one 16-byte store
        *reinterpret_cast<float4 *>(slot + 4 * col) =
            make_float4(acl[0] + acs[0], acl[1] + acs[1], acl[2] + acs[2], acl[3] + acs[3]);
    }
  }
}

// The value of quad lane QP & 3 (DPP quad_perm broadcast).
template <int QP>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, QP, 0xf, 0xf, false);
}

constexpr int FRAG_PAD = 16;

// Wave-wide sum (a float) and maximum (of non-negative floats, compared as
// integers) with DPP alone: row reductions, then row_bcast:15 / :31 carry
// rows 0-2 into row 3, whose lane 63 ends with the result.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_rows(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xf, false);
}
__device__ __forceinline__ float wave_sum63(float v) {
  v = row_sum(v);
  v += __builtin_bit_cast(float, dpp_rows<0x142, 0xa>(__builtin_bit_cast(int, v)));   // row_bcast:15
  v += __builtin_bit_cast(float, dpp_rows<0x143, 0xc>(__builtin_bit_cast(int, v)));   // row_bcast:31
  return lane_f(v, 63);
}
__device__ __forceinline__ float wave_max63_nonneg(float v) {
  unsigned u = __float_as_uint(v);
  u = max(u, (unsigned)dpp_rows<0xb1, 0xf>((int)u));    // quad_perm [1,0,3,2]
  u = max(u, (unsigned)dpp_rows<0x4e, 0xf>((int)u));    // quad_perm [2,3,0,1]
  u = max(u, (unsigned)dpp_rows<0x141, 0xf>((int)u));   // row_half_mirror
  u = max(u, (unsigned)dpp_rows<0x140, 0xf>((int)u));   // row_mirror
  u = max(u, (unsigned)dpp_rows<0x142, 0xa>((int)u));   // row_bcast:15
  u = max(u, (unsigned)dpp_rows<0x143, 0xc>((int)u));   // row_bcast:31
  return __uint_as_float((unsigned)__builtin_amdgcn_readlane((int)u, 63));
}

// W (code bits) is a template parameter: the bit position -> coordinate
// arithmetic of every coefficient then folds to shifts and constants, with
// only the lane's group g and byte t left at run time.
template <int W>
__global__ void __launch_bounds__(256) prep_frag_kernel(PrepGemmArgs a) {
  // per wave: 4 heads x one row each: the dP rotated coordinates any code
  // bit of the record words can name (zero past d), then the mP sketch rows
  // (zero past m), then FRAG_PAD floats (spreads the LDS banks); sized at launch
  extern __shared__ float prs[];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t gx = (int64_t)blockIdx.x * 4 + wv;
  if (gx >= a.groups) return;                       // no block-wide synchronisation below
  const int cwpl = a.cb16, swpl = a.sb16;
  const int d = a.d, m = a.m, dm = d + m;
  const int dP = (128 * cwpl + W - 1) / W, mP = 128 * swpl, ps = dP + mP + FRAG_PAD;
  float *pr = prs + wv * 4 * ps;
  uint8_t *out = a.ws + gx * prep_stride(a.nm);
  const float4 *proj = reinterpret_cast<const float4 *>(out);   // [column][head]
  for (int c = lane; c < dP + mP; c += 64) {
    const int src = c < dP ? (c < d ? c : -1) : (c - dP < m ? d + c - dP : -1);
    const float4 v = src >= 0 ? proj[src] : make_float4(0.f, 0.f, 0.f, 0.f);
    pr[c] = v.x;
    pr[ps + c] = v.y;
    pr[2 * ps + c] = v.z;
    pr[3 * ps + c] = v.w;
  }
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
  // per head: sums of the projections; largest |coefficient| 2^-j over the
  // code (and parity) bits and over the sign bits (j = the bit's place in its byte)
  float sP[4] = {0.f, 0.f, 0.f, 0.f}, sQ[4] = {0.f, 0.f, 0.f, 0.f};
  float mP4[4] = {0.f, 0.f, 0.f, 0.f}, mQ4[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i = lane; i < d; i += 64) {
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      const float v = pr[hh * ps + i], av = fabsf(v);
      sP[hh] += v;
#pragma unroll
      for (int p = 0; p < W; ++p) mP4[hh] = fmaxf(mP4[hh], ldexpf(fabsf(cb2[p]) * av, -((i * W + p) & 7)));
      if constexpr (W == 3) mP4[hh] = fmaxf(mP4[hh], ldexpf(fabsf(cb2[3]) * av, -((3 * i) & 7)));
    }
  }
  for (int jj = lane; jj < m; jj += 64) {
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      const float v = pr[hh * ps + dP + jj];
      sQ[hh] += v;
      mQ4[hh] = fmaxf(mQ4[hh], ldexpf(2.f * fabsf(v), -(jj & 7)));
    }
  }
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    sP[hh] = wave_sum63(sP[hh]);
    sQ[hh] = wave_sum63(sQ[hh]);
    mP4[hh] = wave_max63_nonneg(mP4[hh]);
    mQ4[hh] = wave_max63_nonneg(mQ4[hh]);
  }
  // lane: fragment row r = 4 head + t of lane group g; it computes the
  // coefficients of byte t of its four dwords
  const int r = lane & 15, g = lane >> 4, hr = r >> 2, t = r & 3;
  const float mx0 = hr == 0 ? mP4[0] : hr == 1 ? mP4[1] : hr == 2 ? mP4[2] : mP4[3];
  const float mx1 = hr == 0 ? mQ4[0] : hr == 1 ? mQ4[1] : hr == 2 ? mQ4[2] : mQ4[3];
  // scales 127 / max from the hardware reciprocal (1 ulp: |U| stays below
  // 127.5 2^21, so the top digit stays within int8)
  const float sc0 = mx0 > 0.f ? 127.f * __builtin_amdgcn_rcpf(mx0) : 1.f;
  const float sc1 = mx1 > 0.f ? 127.f * __builtin_amdgcn_rcpf(mx1) : 1.f;
  const float *qr = pr + hr * ps, *qs = qr + dP;
  const int nmc = 2 * cwpl, nmp = 2 * parity_words(cwpl, W);
  // byte selector: byte t of the low operand, byte t of the high operand
  const uint32_t psel = (uint32_t)t | ((uint32_t)(4 + t) << 8) | 0x0c0c0000u;
  wave_sync();                                      // every lane has read the slot
  for (int mu = 0; mu < a.nm; ++mu) {               // (mu, kind, pair, half: the same in every lane)
    const int kind = mu < nmc ? 0 : mu < nmc + nmp ? 1 : 2;   // code bits, merged parity bits, sign bits
    const int mloc = kind == 0 ? mu : kind == 1 ? mu - nmc : mu - nmc - nmp;
    const int wpl = kind == 2 ? swpl : cwpl;
    const float S = kind == 2 ? sc1 : sc0;
    const int pair = mloc >> 1, half = mloc & 1;
    uint32_t dig[4];                               // [e]: the four digits of byte t's coefficient
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = 4 * half + e, q = 8 * t + j;
      float v = 0.f;
      // (the rows are zero past d and m, so no range checks)
      if (kind == 2) {
        const int bitpos = 32 * (g * wpl + pair) + q;
        v = 2.f * qs[bitpos];
      } else if (kind == 0) {
        const int bitpos = 32 * (g * wpl + pair) + q;
        // bitpos / W: a shift, or (W = 3) exact below 2^15 by multiply
        const int i = W == 1 ? bitpos : W == 2 ? bitpos >> 1 : (bitpos * 43691) >> 17;
        // the code bit's plane: j's parity for W = 2 (32 (...) + 8 t is even)
        const float cf = W == 1 ? cb2[0] : W == 2 ? ((e & 1) ? cb2[1] : cb2[0])
                                       : (bitpos - 3 * i == 0 ? cb2[0] : bitpos - 3 * i == 1 ? cb2[1] : cb2[2]);
        v = cf * qr[i];
      } else if constexpr (W == 3) {
        // merged parity word `pair`: bit q belongs to the code starting at bit
        // q of record word g*wpl + p, p = 3 pair + ((q - g*wpl) mod 3)
        const int p = 3 * pair + ((q - g * wpl) % 3 + 3) % 3;
        if (p < wpl) {
          const int bitpos = 32 * (g * wpl + p) + q;
          const int i = (bitpos * 43691) >> 17;
          if (bitpos - 3 * i == 0) v = cb2[3] * qr[i];
        }
      }
      // U = u 2^21 rounded, u = v S 2^-j (negated for j = 7: the B byte value
      // is -128), split into balanced base-128 digits U = r0 2^21 + r1 2^14 +
      // r2 2^7 + r3, |r1|, |r2| <= 64, r3 in [-64, 64)
      const float sj = __builtin_amdgcn_ldexpf((e == 3 && half) ? -S : S, 21 - j);
      const int U = (int)rintf(v * sj);
      const int r0 = (U + (1 << 20)) >> 21;
      const int R1 = U - (r0 << 21);
      const int r1 = (R1 + (1 << 13)) >> 14;
      const int R2 = R1 - (r1 << 14);
      const int r2 = (R2 + 64) >> 7;
      const int r3 = R2 - (r2 << 7);
      // the four low bytes side by side
      dig[e] = __builtin_amdgcn_perm(__builtin_amdgcn_perm((uint32_t)r3, (uint32_t)r2, 0x0c0c0400u),
                                     __builtin_amdgcn_perm((uint32_t)r1, (uint32_t)r0, 0x0c0c0400u), 0x05040100u);
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
    const float xp = lane == 0 ? mP4[0] : lane == 1 ? mP4[1] : lane == 2 ? mP4[2] : mP4[3];
    const float xq = lane == 0 ? mQ4[0] : lane == 1 ? mQ4[1] : lane == 2 ? mQ4[2] : mQ4[3];
    const float s0 = lane == 0 ? sP[0] : lane == 1 ? sP[1] : lane == 2 ? sP[2] : sP[3];
    const float s1 = lane == 0 ? sQ[0] : lane == 1 ? sQ[1] : lane == 2 ? sQ[2] : sQ[3];
    const float bsum = a.basis[0] + (W >= 2 ? a.basis[1] : 0.f) + (W >= 3 ? a.basis[2] + a.basis[3] : 0.f);
    float *cst = reinterpret_cast<float *>(out + (int64_t)a.nm * 1024);
    cst[lane * 4 + 0] = xp > 0.f ? xp * (1.f / 127.f) : 1.f;   // 1 / S, as the scales above
    cst[lane * 4 + 1] = xq > 0.f ? xq * (1.f / 127.f) : 1.f;
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
  a.q16 = ((uintptr_t)q & 15) == 0;
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
  const int pg = 4 * proj_waves(nk);                 // groups per projection block
  const int64_t pblocks = (groups + pg - 1) / pg, fblocks = (groups + 3) / 4;
  if (pblocks > 0x7fffffff || fblocks > 0x7fffffff || a.d + a.m > 512) return TQ_ENOTSUP;
  if (nk <= 4)
    prep_proj_kernel<4><<<(unsigned)pblocks, 64 * proj_waves(4), 0, stream>>>(a);
  else if (nk <= 8)
    prep_proj_kernel<8><<<(unsigned)pblocks, 64 * proj_waves(8), 0, stream>>>(a);
  else
    return TQ_ENOTSUP;
  if (hip_status() != TQ_OK) return TQ_EHIP;
  // (one row per head and wave: dP + mP <= 256 + 256 floats at d <= 256)
  const size_t flds = sizeof(float) * 4 * 4 *
                      (size_t)((128 * a.cb16 + a.w - 1) / a.w + 128 * a.sb16 + FRAG_PAD);   // <= 33 KB
  if (a.w == 1)
    prep_frag_kernel<1><<<(unsigned)fblocks, 256, flds, stream>>>(a);
  else if (a.w == 2)
    prep_frag_kernel<2><<<(unsigned)fblocks, 256, flds, stream>>>(a);
  else
    prep_frag_kernel<3><<<(unsigned)fblocks, 256, flds, stream>>>(a);
  return hip_status();
}

}  // namespace tq
