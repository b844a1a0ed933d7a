// Query prep for many query groups at once (prefill-shaped calls: thousands
// of queries against one key set), d <= 256.  The projections q_rot = Pi q
// and q_s = S q of the estimator (hao.cnyes.com "TurboQuant", 1 bit 掃尾;
// suzuke blog, 第三步) are one GEMM, Q [queries x d] times [Pi; S]^T
// [d x (d + m)], on v_mfma_f32_16x16x32_bf16 with both operands split into
// three bf16 parts (x = x_h + x_m + x_l, each part the bf16 rounding of what
// the previous ones leave) and the six products of order <= 2 accumulated in
// fp32 (h h, h m, m h, m m, h l, l h): about 2^-26 relative error per
// product, as fp32 FMA.  (A two-part split leaves ~2^-17, which moves logits
// near zero by more than the estimator's 1e-4 absolute tolerance.)  Then per
// group of 4 heads: per-head sums and scaled maxima, and the int8 A fragments.
// In a quad of lanes (rows 4 head + digit of one lane group) lane t computes
// the coefficients of byte t of its four dwords and all four base-128 digits
// of each; a byte transpose across the quad (DPP moves and byte selects) then
// gives every lane its own digit of the four bytes.
//
// d <= 128 and code width <= 2 bits: one launch (prep_fused_kernel), the
// projections kept in LDS.  Otherwise two launches:
//  proj: one GEMM per block of 64 queries.  Each wave holds one 16-query
//    tile of A in registers; the [Pi; S] fragments of several 16-column
//    tiles at a time are staged in LDS and shared by the block's waves.  The
//    projections of a group of 4 heads go to the group's own workspace slot
//    (nm KB >= 16 (d + m) bytes).
//  frag: one wave per group of 4 heads: the projections into LDS, then the
//    fragments over the slot.
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

// Coordinates per head row of the fragment kernel's LDS: every coordinate a
// code bit of the record words can name, rounded up to 4 (16-byte reads of
// the sketch rows that follow)
__host__ __device__ constexpr int frag_dp(int cb16, int w) { return ((128 * cb16 + w - 1) / w + 3) & ~3; }

// Balanced base-128 digits of U = rint(x s): the bytes r3, r2, r1, r0 of
// U = r0 2^21 + r1 2^14 + r2 2^7 + r3 with r1, r2, r3 in [-64, 64) (|U| below
// 127.5 2^21 keeps r0 within int8).  Adding 64 (1 + 2^7 + 2^14) makes the three
// low 7-bit fields r + 64 with no borrow between them; flipping their bit 6
// turns each into r in 7-bit two's complement; three bit-field merges of the
// word with itself shifted by one move field k up by k bits, and each copies
// the field's sign bit into bit 7 of its byte.
template <uint32_t MASK>
__device__ __forceinline__ uint32_t merge_shifted(uint32_t y) {   // (y & MASK) | ((y << 1) & ~MASK)
  uint32_t r;
  __asm__("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(MASK), "v"(y), "v"(y << 1));
  return r;
}
__device__ __forceinline__ uint32_t b128_digits(float x, float s) {
  const uint32_t X = (uint32_t)(int)__builtin_rintf(__builtin_fmaf(x, s, 1056832.f)) ^ 0x102040u;
  return merge_shifted<0x7fffffu>(merge_shifted<0x7fffu>(merge_shifted<0x7fu>(X)));
}

// Byte transpose within each quad of lanes, bytes of the input reversed:
// byte c of quad lane l's result is byte 3 - l of quad lane c's input.  Two
// exchange steps (lanes l ^ 1, then l ^ 2), each a DPP move and a byte
// select; sel1 / sel2 are the lane's selectors (l odd: 0x00040206, else
// 0x05010703; l & 2: 0x03020706, else 0x05040100).
__device__ __forceinline__ uint32_t quad_byte_transpose(uint32_t v, uint32_t sel1, uint32_t sel2) {
  const uint32_t p1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xb1, 0xf, 0xf, false);   // quad_perm [1,0,3,2]
  v = __builtin_amdgcn_perm(p1, v, sel1);
  const uint32_t p2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4e, 0xf, 0xf, false);   // quad_perm [2,3,0,1]
  return __builtin_amdgcn_perm(p2, v, sel2);
}

// A DPP move across the rows ROWS (row mask) of the wave, 0 where a row is
// masked off.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_rows(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xf, false);
}

// Eight wave-wide sums and eight wave-wide maxima (of non-negative floats,
// compared as integers) with DPP alone: row reductions, then row_bcast:15 /
// :31 carry rows 0-2 into row 3, whose lane 63 ends with the results.  Each
// step is taken for all sixteen values before the next, so a value's step
// comes fifteen instructions after its previous one, with no wait states.
template <int CTRL, int ROWS>
__device__ __forceinline__ void reduce_step16(float (&s)[8], unsigned (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    s[i] += __builtin_bit_cast(float, dpp_rows<CTRL, ROWS>(__builtin_bit_cast(int, s[i])));
    x[i] = max(x[i], (unsigned)dpp_rows<CTRL, ROWS>((int)x[i]));
  }
}
__device__ __forceinline__ void wave_reduce16(float (&s)[8], unsigned (&x)[8]) {
  reduce_step16<0xb1, 0xf>(s, x);    // quad_perm [1,0,3,2]
  reduce_step16<0x4e, 0xf>(s, x);    // quad_perm [2,3,0,1]
  reduce_step16<0x141, 0xf>(s, x);   // row_half_mirror
  reduce_step16<0x140, 0xf>(s, x);   // row_mirror
  reduce_step16<0x142, 0xa>(s, x);   // row_bcast:15
  reduce_step16<0x143, 0xc>(s, x);   // row_bcast:31
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    s[i] = lane_f(s[i], 63);
    x[i] = (unsigned)__builtin_amdgcn_readlane((int)x[i], 63);
  }
}

// Orders a wave's LDS writes before its reads by other lanes (and its reads
// of a memory range before the range is overwritten).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The int8 A fragments and constants of one group of 4 heads, by one wave,
// from the group's projections in LDS: pr holds 4 rows (one per head, ps
// floats apart) of the dP rotated coordinates any code bit of the record
// words can name (zero past d), then the mP sketch rows (zero past m).
// W (code bits) is a template parameter: the bit position -> coordinate
// arithmetic of every coefficient then folds to shifts and constants, with
// only the lane's group g and byte t left at run time.
template <int W>
__device__ __forceinline__ void frag_group(const PrepGemmArgs &a, const float *pr, int ps, int dP, uint8_t *out,
                                           int lane) {
  const int cwpl = a.cb16, swpl = a.sb16, d = a.d, m = a.m;
  float cb2[4];                                     // 2 basis[p]
#pragma unroll
  for (int p = 0; p < 4; ++p) cb2[p] = 2.f * a.basis[p];
  // per head: sums of the projections; largest |coefficient| 2^-j over the
  // code (and parity) bits and over the sign bits (j = the bit's place in its
  // byte).  A lane's coordinates i = lane + 64 k put their bits at the same
  // places j for every k, so the factors 2^-j |2 basis[plane]| are lane constants.
  float fP = 0.f;
#pragma unroll
  for (int p = 0; p < W; ++p) fP = fmaxf(fP, __builtin_amdgcn_ldexpf(fabsf(cb2[p]), -((lane * W + p) & 7)));
  if constexpr (W == 3) fP = fmaxf(fP, __builtin_amdgcn_ldexpf(fabsf(cb2[3]), -((3 * lane) & 7)));
  const float fQ = __builtin_amdgcn_ldexpf(2.f, -(lane & 7));
  float sP[4] = {0.f, 0.f, 0.f, 0.f}, sQ[4] = {0.f, 0.f, 0.f, 0.f};
  float mP4[4] = {0.f, 0.f, 0.f, 0.f}, mQ4[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i = lane; i < d; i += 64) {
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      const float v = pr[hh * ps + i];
      sP[hh] += v;
      mP4[hh] = fmaxf(mP4[hh], fabsf(v) * fP);
    }
  }
  for (int jj = lane; jj < m; jj += 64) {
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      const float v = pr[hh * ps + dP + jj];
      sQ[hh] += v;
      mQ4[hh] = fmaxf(mQ4[hh], fabsf(v) * fQ);
    }
  }
  {
    float sv[8];
    unsigned xv[8];
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      sv[hh] = sP[hh];
      sv[4 + hh] = sQ[hh];
      xv[hh] = __float_as_uint(mP4[hh]);
      xv[4 + hh] = __float_as_uint(mQ4[hh]);
    }
    wave_reduce16(sv, xv);
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      sP[hh] = sv[hh];
      sQ[hh] = sv[4 + hh];
      mP4[hh] = __uint_as_float(xv[hh]);
      mQ4[hh] = __uint_as_float(xv[4 + hh]);
    }
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
  // coefficient scales of bit j of a byte: S 2^(21 - j), negated for j = 7
  // (that B byte reads -128); the code bits' factor 2 basis[plane] folded in
  // where j fixes the plane (W <= 2), the sign bits' factor 2 always
  float tc[8], ts[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float cf = W == 1 ? cb2[0] : W == 2 ? cb2[j & 1] : 1.f;
    tc[j] = cf * __builtin_amdgcn_ldexpf(j == 7 ? -sc0 : sc0, 21 - j);
    ts[j] = 2.f * __builtin_amdgcn_ldexpf(j == 7 ? -sc1 : sc1, 21 - j);
  }
  const uint32_t sel1 = (t & 1) ? 0x00040206u : 0x05010703u;
  const uint32_t sel2 = (t & 2) ? 0x03020706u : 0x05040100u;
  // fragment mu = (pair, half): byte t of dword e holds bit q = 8 t + 4 half + e
  // of record word (g, pair); the lane computes those four coefficients and
  // their digits (r3 .. r0 in bytes 0 .. 3), and the quad transpose hands
  // digit r_t' (weight 2^(21 - 7 t')) of each to quad lane t'
  uint4 *frag = reinterpret_cast<uint4 *>(out) + lane;
  auto emit = [&](int mu, float x0, float x1, float x2, float x3, const float *tj) {
    const uint32_t d0 = b128_digits(x0, tj[0]), d1 = b128_digits(x1, tj[1]);
    const uint32_t d2 = b128_digits(x2, tj[2]), d3 = b128_digits(x3, tj[3]);
    frag[mu * 64] = make_uint4(quad_byte_transpose(d0, sel1, sel2), quad_byte_transpose(d1, sel1, sel2),
                               quad_byte_transpose(d2, sel1, sel2), quad_byte_transpose(d3, sel1, sel2));
  };
  wave_sync();                                      // every lane has read the slot
  const int nmc = 2 * cwpl, nmp = 2 * parity_words(cwpl, W);
  // (the rows are zero past d and m, so no range checks)
  for (int pair = 0; pair < cwpl; ++pair) {         // code bits
    if constexpr (W == 1) {
      const float *src = qr + 32 * (g * cwpl + pair) + 8 * t;
      const float4 lo = *reinterpret_cast<const float4 *>(src), hi = *reinterpret_cast<const float4 *>(src + 4);
      emit(2 * pair, lo.x, lo.y, lo.z, lo.w, tc);
      emit(2 * pair + 1, hi.x, hi.y, hi.z, hi.w, tc + 4);
    } else if constexpr (W == 2) {
      // bit q of the word is plane (q & 1) of coordinate 16 (g cwpl + pair) + q / 2
      const float4 v = *reinterpret_cast<const float4 *>(qr + 16 * (g * cwpl + pair) + 4 * t);
      emit(2 * pair, v.x, v.x, v.y, v.y, tc);
      emit(2 * pair + 1, v.z, v.z, v.w, v.w, tc + 4);
    } else {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // bitpos / 3 exact below 2^15 by multiply; the remainder is the plane
          const int bitpos = 32 * (g * cwpl + pair) + 8 * t + 4 * half + e;
          const int i = (bitpos * 43691) >> 17, pl = bitpos - 3 * i;
          x[e] = (pl == 0 ? cb2[0] : pl == 1 ? cb2[1] : cb2[2]) * qr[i];
        }
        emit(2 * pair + half, x[0], x[1], x[2], x[3], tc + 4 * half);
      }
    }
  }
  if constexpr (W == 3) {
    for (int pair = 0; pair < nmp / 2; ++pair) {    // merged parity bits
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // bit q of merged word `pair` belongs to the code starting at bit q
          // of record word g*cwpl + p, p = 3 pair + ((q - g*cwpl) mod 3)
          const int q = 8 * t + 4 * half + e;
          const int p = 3 * pair + ((q - g * cwpl) % 3 + 3) % 3;
          const int bitpos = 32 * (g * cwpl + p) + q;
          const int i = (bitpos * 43691) >> 17;
          const bool on = p < cwpl && bitpos == 3 * i;
          x[e] = on ? cb2[3] * qr[on ? i : 0] : 0.f;
        }
        emit(nmc + 2 * pair + half, x[0], x[1], x[2], x[3], tc + 4 * half);
      }
    }
  }
  for (int pair = 0; pair < swpl; ++pair) {         // sign bits: bit q of the word is sketch row 32 (g swpl + pair) + q
    const float *src = qs + 32 * (g * swpl + pair) + 8 * t;
    const float4 lo = *reinterpret_cast<const float4 *>(src), hi = *reinterpret_cast<const float4 *>(src + 4);
    emit(nmc + nmp + 2 * pair, lo.x, lo.y, lo.z, lo.w, ts);
    emit(nmc + nmp + 2 * pair + 1, hi.x, hi.y, hi.z, hi.w, ts + 4);
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

// One wave per group of 4 heads: the group's projections from its workspace
// slot into LDS, then its fragments over the same slot.
template <int W>
__global__ void __launch_bounds__(256) prep_frag_kernel(PrepGemmArgs a) {
  // per wave: 4 heads x one row each (the layout frag_group reads), then
  // FRAG_PAD floats (spreads the LDS banks); sized at launch
  extern __shared__ float prs[];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t gx = (int64_t)blockIdx.x * 4 + wv;
  if (gx >= a.groups) return;                       // no block-wide synchronisation below
  const int d = a.d, m = a.m;
  const int dP = frag_dp(a.cb16, W), mP = 128 * a.sb16, ps = dP + mP + FRAG_PAD;
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
  wave_sync();
  frag_group<W>(a, pr, ps, dP, out, lane);
}

// Query prep of many groups in one launch where d <= 128 and d + m <= 256
// (four k-blocks, sixteen column tiles of [Pi; S]): each of the block's 16
// waves keeps the three bf16 parts of one column tile in registers; per pass
// the block splits 64 query rows (16 groups) into A fragments in LDS, every
// wave multiplies the four A tiles by its column tile into the projection
// rows of the 16 groups in LDS (the layout frag_group reads), and then each
// wave makes one group's fragments.  The projections never go to memory:
// the launch reads the queries and writes the fragments.
constexpr int FUSED_GROUPS = 16;                     // groups per pass (64 query rows)
constexpr int FUSED_PASSES = 4;                      // passes per block (the B registers are loaded once)
constexpr int FUSED_PS = 272;                        // LDS row length: dP + mP + FRAG_PAD at d <= 128
constexpr int FUSED_GS = 4 * FUSED_PS + 16;          // LDS floats per group (16 apart in the banks)

// (at W = 3 the fragment phase's registers and the column tile's 48 do not
// fit the 128 of a 1024-thread block: that width takes the two launches)
__host__ __device__ constexpr bool prep_fused_fits(int nk, int ntile, int w) { return nk <= 4 && ntile <= 16 && w <= 2; }

template <int W>
__global__ void __launch_bounds__(1024) prep_fused_kernel(PrepGemmArgs a) {
  // A fragments of the pass: [A tile][k-block][part h/m/l][lane]
  __shared__ __align__(16) Frag As[4][4][3][64];
  // projections of the pass: [group (FUSED_GS floats)][head][FUSED_PS]
  extern __shared__ float Pt[];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r = lane & 15, g = lane >> 4;
  const int d = a.d, m = a.m, nk = a.nk;
  const int dP = frag_dp(a.cb16, W);
  constexpr int ps = FUSED_PS;
  // B: column tile wv (rows 16 wv + r of [Pi; S]), k-group g
  const bool colw = wv < a.ntile;
  bf16x8 Bh[4], Bm[4], Bl[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int64_t fi = ((int64_t)(colw ? wv : 0) * nk + (kb < nk ? kb : 0)) * 64 + lane;
    Bh[kb] = as_bf(a.MH[fi]);
    Bm[kb] = as_bf(a.MM[fi]);
    Bl[kb] = as_bf(a.ML[fi]);
  }
  // (waited for here: the compiler would otherwise wait inside the pass loop
  // for everything issued before a first use, the prefetched queries included)
  wait_vm<0>();
  // zero the projection rows (columns [d, dP) and past m stay zero)
  {
    float4 *pz = reinterpret_cast<float4 *>(Pt);
    for (int i = tid; i < FUSED_GROUPS * FUSED_GS / 4; i += 1024) pz[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // the thread's A fragment slot: A tile qt, k-block kb, fragment lane fl =
  // row fl & 15 of the tile (query row 16 qt + (fl & 15): group of the pass
  // crow / 4, head crow % 4) and coordinates 32 kb + 8 (fl >> 4) .. + 7
  // (d % 8 == 0: all in or all out); a wave writes 64 consecutive slots
  const int fq = tid >> 8, fk = (tid >> 6) & 3, fl = tid & 63;
  const int crow = 16 * fq + (fl & 15), c0 = 32 * fk + 8 * (fl >> 4);
  const bool chunk = fk < nk;
  auto load_chunk = [&](int64_t gb, float4 &x0, float4 &x1) {
    const int64_t gidx = gb + crow / 4;
    const int64_t grp = gidx / a.hg;
    const int h = (int)(gidx - grp * a.hg) * 4 + crow % 4;
    const int64_t flat = grp * a.qpg + h;
    const bool live = chunk && c0 < d && gidx < a.groups && h < a.qpg && flat < a.nq_total;
    const float *src = a.q + (live ? flat * d + c0 : 0);
    if (!live) {
      x0 = x1 = make_float4(0.f, 0.f, 0.f, 0.f);
    } else if (a.q16) {
      x0 = reinterpret_cast<const float4 *>(src)[0];
      x1 = reinterpret_cast<const float4 *>(src)[1];
    } else {
      x0 = make_float4(src[0], src[1], src[2], src[3]);
      x1 = make_float4(src[4], src[5], src[6], src[7]);
    }
  };
  const int64_t gfirst = (int64_t)blockIdx.x * FUSED_PASSES * FUSED_GROUPS;
  float4 x0, x1;
  load_chunk(gfirst, x0, x1);
  wait_vm<0>();
  for (int pass = 0; pass < FUSED_PASSES; ++pass) {
    const int64_t gb = gfirst + (int64_t)pass * FUSED_GROUPS;
    if (gb >= a.groups) break;                       // (the same in every wave)
    // 1. the chunk as three bf16 parts into its A fragment slot
    if (chunk) {
      const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      bf16x8 ph, pm, pl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ph[e] = (__bf16)xs[e];
        const float r1 = xs[e] - (float)ph[e];        // exact in fp32
        pm[e] = (__bf16)r1;
        pl[e] = (__bf16)(r1 - (float)pm[e]);
      }
      Frag *dst = &As[fq][fk][0][fl];
      dst[0] = __builtin_bit_cast(Frag, ph);
      dst[64] = __builtin_bit_cast(Frag, pm);
      dst[128] = __builtin_bit_cast(Frag, pl);
    }
    __syncthreads();                                 // A written; the previous pass's rows all read
    if (pass + 1 < FUSED_PASSES) load_chunk(gb + FUSED_GROUPS, x0, x1);   // the next pass's chunk, in flight
    // 2. the wave's column tile for the four A tiles
    if (colw) {
      const int c = 16 * wv + r;
      const int pos = c < d ? c : c < d + m ? dP + c - d : -1;
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        f32x4 acs = f32x4{0.f, 0.f, 0.f, 0.f}, acl = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          if (kb >= nk) break;
          const bf16x8 ah = as_bf(As[qt][kb][0][lane]), am = as_bf(As[qt][kb][1][lane]),
                       al = as_bf(As[qt][kb][2][lane]);
          acs = mfma(ah, Bl[kb], acs);
          acl = mfma(ah, Bm[kb], acl);
          acs = mfma(al, Bh[kb], acs);
          acl = mfma(am, Bh[kb], acl);
          acs = mfma(am, Bm[kb], acs);
          acl = mfma(ah, Bh[kb], acl);
        }
        // D rows 4 g + jj of A tile qt: group 4 qt + g, head jj
        if (pos >= 0) {
          float *row = Pt + (4 * qt + g) * FUSED_GS + pos;
          row[0] = acl[0] + acs[0];
          row[ps] = acl[1] + acs[1];
          row[2 * ps] = acl[2] + acs[2];
          row[3 * ps] = acl[3] + acs[3];
        }
      }
    }
    // the next chunk has arrived by now; waiting here rather than at its use
    // keeps that wait from covering the fragment stores issued in between
    wait_vm<0>();
    __syncthreads();                                 // projection rows written; A all read
    // 3. group wv of the pass
    if (gb + wv < a.groups) frag_group<W>(a, Pt + wv * FUSED_GS, ps, dP, a.ws + (gb + wv) * prep_stride(a.nm), lane);
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
  if (prep_fused_fits(nk, a.ntile, a.w)) {
    const int64_t blocks = (groups + FUSED_PASSES * FUSED_GROUPS - 1) / (FUSED_PASSES * FUSED_GROUPS);
    const size_t lds = sizeof(float) * FUSED_GROUPS * FUSED_GS;
    if (blocks > 0x7fffffff || frag_dp(a.cb16, a.w) + 128 * a.sb16 + FRAG_PAD > FUSED_PS) return TQ_ENOTSUP;
    const void *fn = a.w == 1 ? (const void *)prep_fused_kernel<1> : (const void *)prep_fused_kernel<2>;
    if (allow_lds(fn, lds) != TQ_OK) return TQ_EHIP;
    if (a.w == 1)
      prep_fused_kernel<1><<<(unsigned)blocks, 1024, lds, stream>>>(a);
    else
      prep_fused_kernel<2><<<(unsigned)blocks, 1024, lds, stream>>>(a);
    return hip_status();
  }
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
  const size_t flds = sizeof(float) * 4 * 4 * (size_t)(frag_dp(a.cb16, a.w) + 128 * a.sb16 + FRAG_PAD);   // <= 34 KB
  if (a.w == 1)
    prep_frag_kernel<1><<<(unsigned)fblocks, 256, flds, stream>>>(a);
  else if (a.w == 2)
    prep_frag_kernel<2><<<(unsigned)fblocks, 256, flds, stream>>>(a);
  else
    prep_frag_kernel<3><<<(unsigned)fblocks, 256, flds, stream>>>(a);
  return hip_status();
}

}  // namespace tq
