// Vectors longer than 256 coordinates (d up to 1024): quantize and query prep.
//
// The kernels for d <= 256 keep a vector's coordinates, its residual and the
// operand fragments in registers; beyond that they do not fit, so here:
//  * quantize: a block stages 16 vectors in LDS as bf16 (hi, lo) MFMA operand
//    fragments; its four waves split the 16-row output tiles of GEMM 1
//    (Y^T = Pi X^T), search the codebook per coordinate, OR the codes into
//    LDS record words and write the residual (hi, lo) as the operand of GEMM 2
//    (Z^T = S' R^T), whose tiles they split again for the sign bits.  The
//    operand fragments of Pi and S' are read from memory (L2), in plain row
//    order.  The arithmetic is that of the register kernel: bf16-exact split
//    products with fp32 accumulation, fp64 norms, the same decision rules
//    (xujun.org note 189244, 第一步：PolarQuant and 第二步：QJL; suzuke blog
//    "turboquant-compressing-ai-consciousness", 第二步 and 第三步).
//  * query prep: the projections q_rot = Pi q and q_s = S q of a 4-head group
//    are computed into LDS, and every bit coefficient of the estimator's A
//    fragments is formed from them where it is needed (the record bit's
//    coordinate and plane), with the digit expansion of the prep for small d.
#include "tq_quantize_body.h"
#include "tq_score_core.h"

namespace tq {
namespace {

struct QBigArgs {
  const void *x;
  int64_t n, ldx, ldr, ntiles;
  uint8_t *codes, *signs;
  float *norms, *rnorms;
  const Frag *PiH, *PiL, *SH, *SL;
  int d, m, dpad, w, code_bytes, sign_bytes;
  float tpos[8], cpos[8];
  // fractional widths: coordinates d/2 .. d-1 take w2-bit codes (tpos2,
  // cpos2), and the codes are stored as bit planes per coordinate quarter
  int frac, w2;
  float tpos2[8], cpos2[8];
  int planes;          // MSE-only records: codes as bit planes of d bits
};

template <bool BF16IN>
__global__ void __launch_bounds__(256) quantize_big_kernel(QBigArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int NK = a.dpad / 32, NT = a.dpad / 16;
  const int cwn = a.code_bytes / 4, swn = a.sign_bytes / 4;
  Frag *xh = reinterpret_cast<Frag *>(smem);                    // [NK][64] x hi
  Frag *xl = xh + NK * 64;                                       // [NK][64] x lo (fp32 input)
  Frag *rh = xl + (BF16IN ? 0 : NK * 64);                        // [NK][64] residual hi
  Frag *rl = rh + NK * 64;                                       // [NK][64] residual lo
  uint32_t *cwl = reinterpret_cast<uint32_t *>(rl + NK * 64);   // [16][cwn] code words
  uint32_t *swl = cwl + 16 * cwn;                                // [16][swn] sign words
  float *vinv = reinterpret_cast<float *>(swl + 16 * swn);       // [16] 1 / (nu * scale)
  float *vnu = vinv + 16;                                        // [16] nu
  float *rsw = vnu + 16;                                         // [4 waves][16] sum of r^2

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, col = lane & 15, grp = lane >> 4;
  const int qd = a.d / 4, wpp = a.d / 128;       // fractional layout: quarter size, words per plane

  for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    // ---- 1: the 16 vectors' lengths (fp64), then their operand fragments;
    // thread t works on vector t >> 4, chunks of 8 coordinates t & 15 + 16 i
    const int v = tid >> 4, part = tid & 15;
    const int64_t vi = tile * 16 + v;
    const bool valid = vi < a.n;
    auto load8 = [&](int c8, float (&xs)[8]) {
#pragma unroll
      for (int e = 0; e < 8; ++e) xs[e] = 0.f;
      if (!valid || 8 * c8 >= a.d) return;
      if constexpr (BF16IN) {
        const Frag f = *reinterpret_cast<const Frag *>(reinterpret_cast<const uint16_t *>(a.x) + vi * a.ldx + 8 * c8);
        const bf16x8 b = as_bf(f);
#pragma unroll
        for (int e = 0; e < 8; ++e) xs[e] = (float)b[e];
      } else {
        const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.x) + vi * a.ldx + 8 * c8);
        const float4 lo4 = p[0], hi4 = p[1];
        xs[0] = lo4.x; xs[1] = lo4.y; xs[2] = lo4.z; xs[3] = lo4.w;
        xs[4] = hi4.x; xs[5] = hi4.y; xs[6] = hi4.z; xs[7] = hi4.w;
      }
    };
    double ss = 0.0;
    for (int c8 = part; c8 < a.dpad / 8; c8 += 16) {
      float xs[8];
      load8(c8, xs);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += (double)xs[e] * (double)xs[e];
    }
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    ss += __shfl_xor(ss, 4);
    ss += __shfl_xor(ss, 8);
    // vectors shorter than 2^-64 are rotated as x * 2^64 (exact), so that no
    // input or product is a float32 denormal and 1/nu cannot overflow
    const float xsc = (ss > 0.0 && ss < 0x1.0p-128) ? 0x1.0p64f : 1.f;
    for (int c8 = part; c8 < a.dpad / 8; c8 += 16) {
      float xs[8];
      load8(c8, xs);
      const int k = c8 >> 2, lanex = v + 16 * (c8 & 3);
      bf16x8 h, l;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float s = xs[e] * xsc;
        h[e] = (__bf16)s;
        l[e] = (__bf16)(s - (float)h[e]);
      }
      xh[k * 64 + lanex] = __builtin_bit_cast(Frag, h);
      if constexpr (!BF16IN) xl[k * 64 + lanex] = __builtin_bit_cast(Frag, l);
    }
    if (part == 0) {
      const double nud = sqrt(ss);
      vnu[v] = (float)nud;
      vinv[v] = nud > 0.0 ? (float)(1.0 / (nud * (double)xsc)) : 0.f;
    }
    for (int i = tid; i < 16 * (cwn + swn); i += 256) cwl[i] = 0u;       // cwl and swl are contiguous
    __syncthreads();

    // ---- 2: GEMM 1 tiles u = wv (mod 4): codes into LDS words, residual as
    // the GEMM-2 operand; lane (col, grp) holds coordinates 16 u + 4 grp + jj
    // of vector col
    const float inv = vinv[col];
    float rs = 0.f;
    for (int u = wv; u < NT; u += 4) {
      // the tile's 16 coordinates lie in one half (d/2 is a multiple of 16)
      const bool second = a.frac && 16 * u >= a.d / 2;
      const int cw = second ? a.w2 : a.w;
      const int half = (1 << cw) / 2;
      const float *tp = second ? a.tpos2 : a.tpos, *cp = second ? a.cpos2 : a.cpos;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int k = 0; k < NK; ++k) {
        const bf16x8 ah = as_bf(a.PiH[(u * NK + k) * 64 + lane]);
        const bf16x8 al = as_bf(a.PiL[(u * NK + k) * 64 + lane]);
        const bf16x8 bx = as_bf(xh[k * 64 + lane]);
        acc = mfma(ah, bx, acc);
        acc = mfma(al, bx, acc);
        if constexpr (!BF16IN) acc = mfma(ah, as_bf(xl[k * 64 + lane]), acc);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int i = 16 * u + 4 * grp + jj;
        const float y = acc[jj] * inv;
        const uint32_t yb = __float_as_uint(y), ab = yb & 0x7fffffffu;
        uint32_t mm = 0;
        float cm = cp[0];
        for (int j = 0; j < half - 1; ++j) {
          const bool gt = __uint_as_float(ab) > tp[j];
          mm += gt ? 1u : 0u;
          cm = gt ? cp[j + 1] : cm;
        }
        // idx = half + mm for y >= +0, its mirror for y <= -0; r = y - c[idx]
        const uint32_t neg = (uint32_t)((int32_t)yb >> 31);
        uint32_t idx = ((uint32_t)half + mm) ^ (neg & (uint32_t)(2 * half - 1));
        float r = y - __uint_as_float(__float_as_uint(cm) | (yb & 0x80000000u));
        if (i >= a.d) {
          idx = 0u;
          r = 0.f;
        }
        rs += r * r;
        if (a.frac) {
          // quarter g holds its w_g bit planes of qd bits each, quarters in order
          const int g = i / qd, jq = i - g * qd;
          const int base = g < 2 ? g * a.w * wpp : 2 * a.w * wpp + (g - 2) * a.w2 * wpp;
          for (int pl = 0; pl < cw; ++pl)
            if ((idx >> pl) & 1u) atomicOr(&cwl[col * cwn + base + pl * wpp + (jq >> 5)], 1u << (jq & 31));
        } else if (a.planes) {
          // MSE-only records: bit pl of code i at record bit pl d + i
          for (int pl = 0; pl < a.w; ++pl) {
            const int bit = pl * a.d + i;
            if ((idx >> pl) & 1u) atomicOr(&cwl[col * cwn + (bit >> 5)], 1u << (bit & 31));
          }
        } else {
          const int bit = i * a.w;
          if (idx) {
            atomicOr(&cwl[col * cwn + (bit >> 5)], idx << (bit & 31));
            if ((bit & 31) + a.w > 32) atomicOr(&cwl[col * cwn + (bit >> 5) + 1], idx >> (32 - (bit & 31)));
          }
        }
        if (a.m > 0) {
          const __bf16 h = (__bf16)r, l = (__bf16)(r - (float)h);
          const int k2 = i >> 5, lane2 = col + 16 * ((i & 31) >> 3), e2 = i & 7;
          reinterpret_cast<__bf16 *>(&rh[k2 * 64 + lane2])[e2] = h;
          reinterpret_cast<__bf16 *>(&rl[k2 * 64 + lane2])[e2] = l;
        }
      }
    }
    rs += __shfl_xor(rs, 16);
    rs += __shfl_xor(rs, 32);
    if (grp == 0) rsw[wv * 16 + col] = rs;
    __syncthreads();

    // ---- 3: GEMM 2 tiles (JL sketch of the residual) -> sign words
    if (a.m > 0) {
      for (int u = wv; u < NT; u += 4) {
        f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int k = 0; k < NK; ++k) {
          const bf16x8 sh = as_bf(a.SH[(u * NK + k) * 64 + lane]);
          const bf16x8 sl = as_bf(a.SL[(u * NK + k) * 64 + lane]);
          const bf16x8 bh = as_bf(rh[k * 64 + lane]), bl = as_bf(rl[k * 64 + lane]);
          z = mfma(sh, bh, z);
          z = mfma(sh, bl, z);
          z = mfma(sl, bh, z);
        }
        // bit = [z >= 0] (sums start at +0, so z is never -0); rows past m are 0
        const int j0 = 16 * u + 4 * grp;
        uint32_t nib = 0u;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) nib |= (j0 + jj < a.m && !(__float_as_uint(z[jj]) >> 31)) ? (1u << jj) : 0u;
        if (nib) atomicOr(&swl[col * swn + (j0 >> 5)], nib << (j0 & 31));
      }
    }
    __syncthreads();

    // ---- 4: records out (a zero vector: zero codes, zero signs, gamma = 0)
    for (int i = tid; i < 16 * cwn; i += 256) {
      const int vv = i / cwn, wd = i - vv * cwn;
      const int64_t vj = tile * 16 + vv;
      if (vj < a.n)
        reinterpret_cast<uint32_t *>(a.codes + vj * a.ldr * a.code_bytes)[wd] = vnu[vv] > 0.f ? cwl[i] : 0u;
    }
    if (a.m > 0) {
      for (int i = tid; i < 16 * swn; i += 256) {
        const int vv = i / swn, wd = i - vv * swn;
        const int64_t vj = tile * 16 + vv;
        if (vj < a.n)
          reinterpret_cast<uint32_t *>(a.signs + vj * a.ldr * a.sign_bytes)[wd] = vnu[vv] > 0.f ? swl[i] : 0u;
      }
    }
    if (tid < 16) {
      const int64_t vj = tile * 16 + tid;
      if (vj < a.n) {
        a.norms[vj * a.ldr] = vnu[tid];
        if (a.m > 0) {
          const float r2 = (rsw[tid] + rsw[16 + tid]) + (rsw[32 + tid] + rsw[48 + tid]);
          a.rnorms[vj * a.ldr] = vnu[tid] > 0.f ? sqrtf(r2) : 0.f;
        }
      }
    }
    __syncthreads();
  }
}

// Query prep for d > 256, in two launches per job:
//  proj: q_rot = Pi q and q_s = S q of every (KV group, 4-head block), one
//        block per group and 64 projection columns (the four waves take a
//        quarter of the rows each), written into the group's own workspace
//        slot (the slot is larger than the projections: nm KB >= 16 (d + m) B);
//  frag: per group, the projections into LDS, then per head the sums and
//        scaled maxima, then the A fragments and constants (the same digit
//        expansion as the prep for small d), over the slot.
struct PrepBigArgs {
  const float *q;      // [G][qpg][d]
  const float *PiT;    // [d][d]
  const float *ST;     // [d][m]
  uint8_t *ws;
  int64_t nq_total;
  int d, m, w, qpg, hg, cb, sb, nm;
  float basis[4];
  int cw16;            // code words per lane group
  int frac, w2;        // fractional widths: the second half's code bits and codebook
  float basis2[4];
};

__global__ void __launch_bounds__(256) proj_big_kernel(PrepBigArgs a) {
  extern __shared__ __align__(16) float4 qT4[];     // [d] x 4 heads
  __shared__ float4 red[4][64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int gidx = blockIdx.x, grp = gidx / a.hg, hgi = gidx - grp * a.hg;
  const int d = a.d, m = a.m;
  float *qT = reinterpret_cast<float *>(qT4);
  for (int i = tid; i < 4 * d; i += 256) {
    const int hh = i / d, j = i - hh * d;
    const int h = hgi * 4 + hh;
    const int64_t flat = (int64_t)grp * a.qpg + h;
    qT[j * 4 + hh] = (h < a.qpg && flat < a.nq_total) ? a.q[flat * d + j] : 0.f;
  }
  __syncthreads();
  const int c = blockIdx.y * 64 + lane;
  const bool isp = c < d;
  const float *MT = isp ? a.PiT : a.ST;
  const int cols = isp ? d : m;
  const int cc = min(isp ? c : c - d, max(cols, 1) - 1);
  const int rows = d / 4, j0 = wv * rows;       // d % 8 == 0
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (c < d + m) {
    for (int j = j0; j < j0 + rows; ++j) {
      const float mv = MT[(int64_t)j * cols + cc];
      const float4 q4 = qT4[j];
      acc.x = fmaf(mv, q4.x, acc.x);
      acc.y = fmaf(mv, q4.y, acc.y);
      acc.z = fmaf(mv, q4.z, acc.z);
      acc.w = fmaf(mv, q4.w, acc.w);
    }
  }
  red[wv][lane] = acc;
  __syncthreads();
  if (wv == 0 && c < d + m) {
    float4 s = red[0][lane];
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      s.x += red[i][lane].x;
      s.y += red[i][lane].y;
      s.z += red[i][lane].z;
      s.w += red[i][lane].w;
    }
    float *proj = reinterpret_cast<float *>(a.ws + (int64_t)gidx * prep_stride(a.nm));
    const int dm = d + m;
    proj[0 * dm + c] = s.x;
    proj[1 * dm + c] = s.y;
    proj[2 * dm + c] = s.z;
    proj[3 * dm + c] = s.w;
  }
}

__global__ void __launch_bounds__(256) frag_big_kernel(PrepBigArgs a) {
  extern __shared__ __align__(16) float pr[];       // [4][d + m]: q_rot then q_s per head
  __shared__ float redall[4][4][4];                 // [wave][head][sP, sQ, mP, mQ]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int gidx = blockIdx.x;
  const int d = a.d, m = a.m, w = a.w, dm = d + m;
  uint8_t *out = a.ws + (int64_t)gidx * prep_stride(a.nm);
  const float *proj = reinterpret_cast<const float *>(out);
  for (int i = tid; i < 4 * dm; i += 256) pr[i] = proj[i];
  __syncthreads();          // the slot is read in full before it is overwritten
  auto qr = [&](int hh, int i) { return pr[hh * dm + i]; };
  auto qs = [&](int hh, int j) { return pr[hh * dm + d + j]; };
  // per head: sums (P: code chain, Q: sign chain) and the largest
  // |coefficient| 2^-(bit & 7) of each chain
  float sP[4] = {0.f, 0.f, 0.f, 0.f}, sQ[4] = {0.f, 0.f, 0.f, 0.f};
  float mP[4] = {0.f, 0.f, 0.f, 0.f}, mQ[4] = {0.f, 0.f, 0.f, 0.f};
  const float bsum1 = a.basis[0] + (w >= 2 ? a.basis[1] : 0.f) + (w >= 3 ? a.basis[2] + a.basis[3] : 0.f);
  const float bsum2 = a.basis2[0] + (a.w2 >= 2 ? a.basis2[1] : 0.f);
  const int qd = d / 4, wpp = d / 128;
  // fractional widths: sum_i (sum of coordinate i's basis) q_rot[i] directly
  for (int i = tid; i < d; i += 256) {
    const float wt = a.frac ? (i < d / 2 ? bsum1 : bsum2) : 1.f;
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) sP[hh] = fmaf(wt, qr(hh, i), sP[hh]);
  }
  for (int j = tid; j < m; j += 256)
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      sQ[hh] += qs(hh, j);
      mQ[hh] = fmaxf(mQ[hh], ldexpf(fabsf(2.f * qs(hh, j)), -(j & 7)));
    }
  if (a.frac) {
    // bit (plane pl, coordinate i) sits at bit (i mod qd) & 7 of its byte
    for (int i = tid; i < d; i += 256) {
      const bool second = i >= d / 2;
      const int cw = second ? a.w2 : w, e = (i % qd) & 7;
      const float *bs = second ? a.basis2 : a.basis;
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        for (int pl = 0; pl < cw; ++pl) mP[hh] = fmaxf(mP[hh], ldexpf(fabsf(2.f * bs[pl] * qr(hh, i)), -e));
        if (cw == 3) mP[hh] = fmaxf(mP[hh], ldexpf(fabsf(2.f * bs[3] * qr(hh, i)), -e));
      }
    }
  } else {
    for (int pos = tid; pos < d * w; pos += 256) {
      const int i = pos / w, p = pos - i * w;
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        mP[hh] = fmaxf(mP[hh], ldexpf(fabsf(2.f * a.basis[p] * qr(hh, i)), -(pos & 7)));
        if (w == 3 && p == 0) mP[hh] = fmaxf(mP[hh], ldexpf(fabsf(2.f * a.basis[3] * qr(hh, i)), -(pos & 7)));
      }
    }
  }
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    const float t0 = wave_sum(sP[hh]), t1 = wave_sum(sQ[hh]), t2 = wave_max(mP[hh]), t3 = wave_max(mQ[hh]);
    if (lane == 0) {
      redall[wv][hh][0] = t0;
      redall[wv][hh][1] = t1;
      redall[wv][hh][2] = t2;
      redall[wv][hh][3] = t3;
    }
  }
  __syncthreads();
  // A fragments: dword (mu * 64 + lane) * 4 + e; thread tid writes dword tid
  // of every mu, so its lane (row -> head, digit) and e are fixed
  const int flane = tid >> 2, e = tid & 3;
  const int row = flane & 15, g = flane >> 4;
  const int hh = row >> 2, digit = row & 3;
  float mx0 = 0.f, mx1 = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mx0 = fmaxf(mx0, redall[i][hh][2]);
    mx1 = fmaxf(mx1, redall[i][hh][3]);
  }
  const float sc0 = mx0 > 0.f ? 127.f / mx0 : 1.f, sc1 = mx1 > 0.f ? 127.f / mx1 : 1.f;
  const int cwpl = a.cw16, swpl = a.sb / 16;
  const int nmc = 2 * cwpl, nmp = 2 * parity_words(cwpl, w);
  for (int mu = 0; mu < a.nm; ++mu) {
    int mloc, wpl, kind;          // kind 0: code bits, 1: merged parity bits, 2: sign bits
    float S;
    if (mu < nmc) {
      kind = 0; mloc = mu; wpl = cwpl; S = sc0;
    } else if (mu < nmc + nmp) {
      kind = 1; mloc = mu - nmc; wpl = cwpl; S = sc0;
    } else {
      kind = 2; mloc = mu - nmc - nmp; wpl = swpl; S = sc1;
    }
    const int pair = mloc >> 1, hlf = mloc & 1;
    const int j = 4 * hlf + e;
    uint32_t dw = 0u;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int q = 8 * b + j;
      // merged parity word `pair`: bit q belongs to the code starting at bit
      // q of record word g*wpl + p, p = 3 pair + ((q - g*wpl) mod 3), if any
      const int p = kind == 1 && !a.frac ? 3 * pair + ((q - g * wpl) % 3 + 3) % 3 : pair;
      const int bitpos = 32 * (g * wpl + p) + q;
      float vcoef = 0.f;
      if (a.frac && kind != 2) {
        // word slot p of lane group g: plane p / wpp of the quarter's
        // coordinates 32 (p mod wpp) .. +31; the parity words (3-bit codes,
        // first half only) are the planes' XOR, one per plane word
        const int cw = g < 2 ? w : a.w2;
        const float *bs = g < 2 ? a.basis : a.basis2;
        const int pl = kind == 0 ? p / wpp : 0, jw = kind == 0 ? p % wpp : p;
        const int i = g * qd + 32 * jw + q;
        if (kind == 0 && pl < cw) vcoef = 2.f * bs[pl] * qr(hh, i);
        if (kind == 1 && cw == 3 && p < wpp) vcoef = 2.f * bs[3] * qr(hh, i);
      } else if (p < wpl) {
        if (kind == 0) {
          const int i = bitpos / w, pl = bitpos - i * w;
          if (i < d) vcoef = 2.f * a.basis[pl] * qr(hh, i);
        } else if (kind == 1) {
          const int i = bitpos / 3;
          if (bitpos - 3 * i == 0 && i < d) vcoef = 2.f * a.basis[3] * qr(hh, i);
        } else if (bitpos < m) {
          vcoef = 2.f * qs(hh, bitpos);
        }
      }
      float u = ldexpf(vcoef * S, -j);
      if (j == 7) u = -u;                 // B byte value is -128 for bit 7
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
    reinterpret_cast<uint32_t *>(out)[mu * 256 + tid] = dw;
  }
  if (tid < 4) {
    const int h4 = tid;
    float s0 = 0.f, s1 = 0.f, x0 = 0.f, x1 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s0 += redall[i][h4][0];
      s1 += redall[i][h4][1];
      x0 = fmaxf(x0, redall[i][h4][2]);
      x1 = fmaxf(x1, redall[i][h4][3]);
    }
    float *cst = reinterpret_cast<float *>(out + (int64_t)a.nm * 1024);
    cst[h4 * 4 + 0] = x0 > 0.f ? 1.f / (127.f / x0) : 1.f;
    cst[h4 * 4 + 1] = x1 > 0.f ? 1.f / (127.f / x1) : 1.f;
    cst[h4 * 4 + 2] = a.frac ? s0 : bsum1 * s0;
    cst[h4 * 4 + 3] = s1;
  }
}

}  // namespace

int launch_quantize_big(const tq_ctx *ctx, const void *x, int dtype, int64_t n, int64_t ldx, int64_t ldr,
                        uint8_t *codes, uint8_t *signs, float *norms, float *rnorms, hipStream_t stream) {
  if (n == 0) return TQ_OK;
  QBigArgs a{};
  a.x = x;
  a.n = n;
  a.ldx = ldx;
  a.ldr = ldr;
  a.ntiles = (n + 15) / 16;
  a.codes = codes;
  a.signs = signs;
  a.norms = norms;
  a.rnorms = rnorms;
  a.PiH = ctx->PiA_hi;
  a.PiL = ctx->PiA_lo;
  a.SH = ctx->S2A_hi;
  a.SL = ctx->S2A_lo;
  a.d = ctx->hp.d;
  a.m = ctx->hp.m;
  a.dpad = ctx->dpad;
  a.w = ctx->hp.w;
  a.code_bytes = ctx->code_bytes;
  a.sign_bytes = ctx->sign_bytes;
  for (int j = 0; j < 8; ++j) {
    a.tpos[j] = ctx->tpos[j];
    a.cpos[j] = ctx->cpos[j];
    a.tpos2[j] = ctx->tpos2[j];
    a.cpos2[j] = ctx->cpos2[j];
  }
  a.frac = ctx->frac;
  a.w2 = ctx->hp.w2;
  a.planes = ctx->hp.mode == TQ_MODE_MSE;
  const bool bf16 = dtype == TQ_BF16;
  const int NK = a.dpad / 32;
  const size_t frag_bytes = sizeof(Frag) * 64 * (size_t)NK * ((bf16 ? 1 : 2) + 2);
  const size_t lds = frag_bytes + 4 * 16 * (size_t)(a.code_bytes / 4 + a.sign_bytes / 4) + 4 * (16 + 16 + 64);
  const int64_t cap = (int64_t)ctx->cus * 2;
  const int blocks = (int)(a.ntiles < cap ? a.ntiles : cap);
  const void *fn = bf16 ? reinterpret_cast<const void *>(&quantize_big_kernel<true>)
                        : reinterpret_cast<const void *>(&quantize_big_kernel<false>);
  if (allow_lds(fn, lds) != TQ_OK) return TQ_EHIP;
  if (bf16)
    quantize_big_kernel<true><<<blocks, 256, lds, stream>>>(a);
  else
    quantize_big_kernel<false><<<blocks, 256, lds, stream>>>(a);
  return hip_status();
}

int launch_prep_big(const tq_ctx *ctx, const float *q, int64_t groups, int qpg, int hg, int64_t nq_total,
                    uint8_t *ws, hipStream_t stream) {
  PrepBigArgs a{};
  a.q = q;
  a.PiT = ctx->PiT32;
  a.ST = ctx->ST32;
  a.ws = ws;
  a.nq_total = nq_total;
  a.d = ctx->hp.d;
  a.m = ctx->hp.m;
  a.w = ctx->hp.w;
  a.qpg = qpg;
  a.hg = hg;
  a.cb = ctx->code_bytes;
  a.sb = ctx->sign_bytes;
  a.nm = mfma_count(ctx->cw16, ctx->sign_bytes / 16, ctx->hp.w);
  for (int i = 0; i < 4; ++i) {
    a.basis[i] = ctx->basis[i];
    a.basis2[i] = ctx->basis2[i];
  }
  a.cw16 = ctx->cw16;
  a.frac = ctx->frac;
  a.w2 = ctx->hp.w2;
  if (groups == 0) return TQ_OK;
  if (groups > 0x7fffffff) return TQ_ENOTSUP;
  const unsigned cblocks = (unsigned)((a.d + a.m + 63) / 64);
  proj_big_kernel<<<dim3((unsigned)groups, cblocks), 256, sizeof(float) * 4 * (size_t)a.d, stream>>>(a);
  if (hip_status() != TQ_OK) return TQ_EHIP;
  frag_big_kernel<<<(unsigned)groups, 256, sizeof(float) * 4 * (size_t)(a.d + a.m), stream>>>(a);
  return hip_status();
}

}  // namespace tq
