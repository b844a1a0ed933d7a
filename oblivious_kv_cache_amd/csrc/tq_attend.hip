// Fused decode attention over a packed KV cache.
//
// Keys are TurboQuant records (scored by the estimator of tq_scores.hip);
// values are MSE-stage records (codes + norm) of a second context; both K and
// V live in the cache (xujun.org note 189244, section KV 缓存).  For one query
// group (<= 4 heads sharing a KV head):
//   z_t   = scale * l_t,   p_t = softmax_t(z),
//   out   = sum_t p_t * nu_t * Pi_v^T c_v[idx_t]
//         = Pi_v^T ( sum_t p_t nu_t c_v[idx_t] )     (rotate back once).
// Split over token chunks like flash-decoding on one GPU:
//   partial kernel (block = one query group x a run of chunks, online softmax):
//     A. int8-MFMA logits of the chunk into LDS (and to the optional logits
//        output); the chunk's value records staged in LDS;
//     B. chunk max, running max M, rescale factor f = exp(M_old - M_new);
//        weights w_t = exp(z_t - M) nu_t turned into int8 fixed-point digits
//        (the A operand of the value sum); the staged value records
//        transposed into bit-plane words (32 tokens per word);
//     C. the value sum on int8 MFMA over bit planes (below);
//     D. per-block partials (M, sum of exp, rotated accumulator).
//   combine kernel: merges the partials with the usual max rescaling,
//     divides by the total, applies Pi_v^T; optionally normalises the logits
//     to probs.
//
// Value sum on matrix cores.  The value codebook is antisymmetric, so a
// centroid is an odd multilinear polynomial of the sign variables
// s_p = 2 bit_p - 1 of its code bits: c = sum_P A_P prod_{p in P} s_p over the
// single bits and (w >= 3) the triples of bits, where a product of three signs
// is 2 (parity of the three bits) - 1.  Hence for coordinate i
//   sum_t w_t c[idx_t,i] = sum_P A_P (2 V_P,i - W),
//   V_P,i = sum_t w_t beta_P(t,i),   W = sum_t w_t,
// with beta_P the bit (or bit parity) P of token t's code i.  V is an int8
// matrix product over tokens: the A operand holds the weights of 64 tokens as
// four base-128 digits per head (16 rows = 4 heads x 4 digits, scaled per
// chunk), the B operand the bits of 64 tokens of 16 coordinates, built from
// one 32-token plane word per lane as (word & 0x01010101 << j) -- bit j of
// each byte -- exactly as the key estimator builds its B from record words.
// The plane words come from the staged value records by 32 x 32 bit
// transposes.  W is the same product against an all-ones B, so 2 V - W is
// exact in int32 before the digits are recombined in fp32.
#include <algorithm>
#include <cfloat>

#include "tq_score_core.h"

namespace tq {
namespace {

constexpr int CH = 512;            // tokens per chunk
constexpr int NT = 256;            // threads per partial block
constexpr int NB32 = CH / 32;      // 32-token plane words per bit row and chunk
#ifndef TQ_ATT_BLOCKS
#define TQ_ATT_BLOCKS 512          // partial blocks per call (2 per CU are resident)
#endif

// odd monomials of the code bits of a w-bit value code: w singles + triples
__host__ __device__ constexpr int value_planes(int vw) { return vw + (vw == 3 ? 1 : vw == 4 ? 4 : 0); }

struct AttArgs {
  const uint8_t *kcodes, *ksigns;
  const float *knorms, *krnorms;
  const uint8_t *vcodes;
  const float *vnorms;
  const uint8_t *prep;
  float *logits;                   // optional [G][qpg][T]
  float *part;                     // [G*hg][nsplit][4][d + 2]
  int64_t T, ldk;
  int qpg, hg, nchunk, nsplit, cps, d, kcb, ksb, vcb;
  float alpha, scale;
  float vbasis[8];                 // value codebook: odd-monomial coefficients
};

// 32 x 32 bit transpose in registers: afterwards bit i of x[q] is what bit q
// of x[i] was.  Five rounds swap the off-diagonal blocks of size J.
template <int J>
__device__ __forceinline__ void transpose_round(uint32_t (&x)[32]) {
  constexpr uint32_t M = J == 4 ? 0x0f0f0f0fu : J == 2 ? 0x33333333u : 0x55555555u;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    if ((k & J) == 0) {
      const uint32_t lo = x[k], hi = x[k + J];
      if constexpr (J == 16) {          // whole 16-bit halves: byte permutes
        x[k] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
        x[k + J] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
      } else if constexpr (J == 8) {    // whole bytes: byte permutes
        x[k] = __builtin_amdgcn_perm(hi, lo, 0x06020400u);
        x[k + J] = __builtin_amdgcn_perm(hi, lo, 0x07030501u);
      } else {                          // bit fields: two bitfield selects
        x[k] = (lo & M) | ((hi << J) & ~M);
        x[k + J] = ((lo >> J) & M) | (hi & ~M);
      }
    }
  }
}
__device__ __forceinline__ void transpose32(uint32_t (&x)[32]) {
  transpose_round<16>(x);
  transpose_round<8>(x);
  transpose_round<4>(x);
  transpose_round<2>(x);
  transpose_round<1>(x);
}

// One block = one query group x one split (a run of `cps` chunks of CH
// tokens).  Wave wv owns the 64-token blocks wv and wv + 4 of every chunk and
// everything computed from them: their logits, staged value records, plane
// words, fixed-point weights and value sums, with an online softmax of its
// own (running max M and sum of exp per head; the value accumulators are
// rescaled by exp(M_old - M_new) whenever its tokens raise the max).  The
// waves therefore never wait for each other inside the chunk loop; their
// four partial softmax states are merged once at the end.  The key words,
// value records and value norms of the wave's next tokens are loaded into
// registers while the current ones are processed.
#ifndef TQ_ATT_WAVES_PER_EU
#define TQ_ATT_WAVES_PER_EU 2
#endif
template <int CB16, int SB16, int W, int VW>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(TQ_ATT_WAVES_PER_EU)))
attend_partial_kernel(AttArgs a) {
  constexpr int NM = ScoreShape<CB16, SB16, W>::NM;
  using KW = KeyWords<CB16, SB16, W>;
  constexpr int NPL = value_planes(VW);
  constexpr int VBMAX = 16 * VW;                  // value record bytes (d <= 128)
  constexpr int VR = VBMAX / 8;                   // 16-byte value units per lane per chunk, at most
  constexpr int NPMAX = VBMAX * 8;                // bit rows of a value record
  constexpr int WT = 128;                         // tokens of a wave per chunk
  // plane-word rows: bit row P of a 32-token block at plane_index(P), a skew
  // of 4 words per coordinate tile (16 VW rows) and a block stride of TSTR
  // words (4 mod 32) spread the LDS banks of both the transposing lanes and
  // the MFMA operand readers; the rows of the next coordinate tile are then
  // 16 VW + 4 words on
  auto plane_index = [](int P) { return P + 4 * (P / (16 * VW)); };
  constexpr int TSTR = NPMAX + NPMAX / (4 * VW) + 4;
  // fixed-point weights U = w S 2^(21 - j), [head][token] with a skew of 4
  // words per 32 tokens
  constexpr int UST = WT + WT / 8 + 4;
  auto uidx = [](int t) { return t + 4 * (t >> 5); };
  struct WaveLds {
    float zt[WT][4];                              // scaled logits [token][head]
    uint32_t vrec[WT * VBMAX / 4];                // staged value records, token-major
    uint32_t tpl[WT / 32 * TSTR];                 // plane words [32-token block][bit row]
    uint32_t ufix[4 * UST];                       // fixed-point weights
    float vacc[4][128 + 16];                      // value sums [head][rotated coordinate]
  };
  __shared__ __align__(16) WaveLds wl[NT / 64];
  __shared__ float fin[NT / 64][4][2];            // per wave and head: running max, sum of exp

  const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, grp = lane >> 4, wv = tid >> 6;
  WaveLds &L = wl[wv];
  const int64_t gidx = blockIdx.y, kg = gidx / a.hg;
  const int hgi = (int)(gidx - kg * a.hg);
  const int c_begin = blockIdx.x * a.cps;
  const int c_end = min(c_begin + a.cps, a.nchunk);
  const int d = a.d;
  const int64_t T = a.T;
  const int vcb = a.vcb, nd = vcb / 4;                 // value record dwords
  const int nct = (d + 15) / 16;                       // 16-coordinate tiles

  const uint8_t *prep = a.prep + gidx * prep_stride(NM);
  i32x4 A[NM];
#pragma unroll
  for (int mu = 0; mu < NM; ++mu) A[mu] = reinterpret_cast<const i32x4 *>(prep)[mu * 64 + lane];
  const float *cst = reinterpret_cast<const float *>(prep + NM * 1024) + grp * 4;
  const HeadConsts hc = HeadConsts::load(cst);
  const ParityMasks<CB16, W> pm = parity_masks<CB16, W>(grp);
  const int head = hgi * 4 + grp;
  const uint8_t *kcb = a.kcodes + kg * a.ldk * a.kcb;
  const uint8_t *ksb = a.ksigns + kg * a.ldk * a.ksb;
  const float *knb = a.knorms + kg * a.ldk, *krb = a.krnorms + kg * a.ldk;
  const uint8_t *vcbp = a.vcodes + kg * a.ldk * a.vcb;
  const float *vnb = a.vnorms + kg * a.ldk;
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

  // registers of the wave's tokens in flight: key words per 16-key subtile,
  // key norms one per lane (handed out by cross-lane reads), the value
  // records of the wave's two 64-token blocks (VR 16-byte units per lane)
  // and the value norms of tokens lane and lane + 64
  KW kw[2][4];
  float knu[2], kga[2], vn[2];
  u32x4 vr[VR];
  const int vunits = 4 * vcb;                        // 16-byte units of a 64-token block
  auto issue = [&](int c) {
    // 32-bit offsets from the group's base pointers (the host checks that a
    // group's records span less than 4 GB) keep the address math short
    const int tlast = (int)T - 1;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tb = c * CH + (wv + 4 * tt) * 64;   // first token of the block
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t t = (uint32_t)min(tb + 16 * s + col, tlast);
        const uint8_t *cp = kcb + (t * (CB16 * 16) + (uint32_t)grp * (CB16 * 4));
        const uint8_t *sp = ksb + (t * (SB16 * 16) + (uint32_t)grp * (SB16 * 4));
#pragma unroll
        for (int i = 0; i < CB16; ++i) kw[tt][s].cw[i] = key_word<true>(reinterpret_cast<const uint32_t *>(cp + 4 * i));
#pragma unroll
        for (int i = 0; i < SB16; ++i) kw[tt][s].sw[i] = key_word<true>(reinterpret_cast<const uint32_t *>(sp + 4 * i));
      }
      const uint32_t tl = (uint32_t)min(tb + lane, tlast);
      knu[tt] = load_f32(knb, tl);
      kga[tt] = load_f32(krb, tl);
      vn[tt] = vnb[tl];
      // value records: clamped 16-byte units (units past the cache end
      // repeat the last real one; their tokens get zero weight)
      const int tbc = min(tb, tlast);              // a block past the cache end reads its last token
      const uint32_t lim = (uint32_t)(min(64, (int)T - tbc) * (vcb / 16)) - 1u;
      const u32x4 *src = reinterpret_cast<const u32x4 *>(vcbp + (uint32_t)tbc * vcb);
#pragma unroll
      for (int b = 0; b < VR / 2; ++b)
        if (b * 64 < vunits) vr[tt * (VR / 2) + b] = __builtin_nontemporal_load(src + min((uint32_t)(b * 64 + lane), lim));
    }
  };

  // B operand masks of the value sum: lane group g takes bits 4 (g & 1) + e
  // of each byte of its plane word (dword e of the operand)
  const int vhalf = grp & 1;
  const uint32_t bm0 = 0x01010101u << (4 * vhalf), bm1 = bm0 << 1, bm2 = bm0 << 2, bm3 = bm0 << 3;
  auto vplanes = [&](uint32_t w) { return i32x4{(int)(w & bm0), (int)(w & bm1), (int)(w & bm2), (int)(w & bm3)}; };
  // within-wave ordering of LDS accesses between lanes (the waves never wait
  // for each other)
  // (the LDS executes a wave's instructions in order, so the compiler only
  // has to keep the accesses on their side of this point)
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  float M[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  float lsum[4] = {0.f, 0.f, 0.f, 0.f};
  float *vac = &L.vacc[grp][col];                  // coordinate 16 ct + col of head grp: vac[16 ct]
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) vac[16 * ct] = 0.f;
  int pr0[VW];
#pragma unroll
  for (int p = 0; p < VW; ++p) pr0[p] = plane_index(col * VW + p);
  // A operand of the value sum: lane (row m = 4 h + digit, group g) holds, at
  // dword e and byte b, digit (m & 3) of head (m >> 2) for the wave's token
  // 64 tt + 32 (g >> 1) + 8 b + 4 (g & 1) + e, negated for bit 7 (B byte -128)
  const int ah = col >> 2, ash = 21 - 7 * (col & 3);

  issue(c_begin);
  for (int c = c_begin; c < c_end; ++c) {
    const int64_t tbeg = (int64_t)c * CH;
    // ---- A: logits of the wave's tokens into LDS; value records staged
    float lg[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if constexpr (W == 3) {   // first code word of the next lane group (lane + 16), none for the last
          const uint32_t nxt = (uint32_t)__shfl((int)kw[tt][s].cw[0], (lane + 16) & 63);
          kw[tt][s].cw[CB16] = grp < 3 ? nxt : 0u;
        }
        const float nu = __shfl(knu[tt], 16 * s + col), ga = __shfl(kga[tt], 16 * s + col);
        lg[tt][s] = tile_logit<CB16, SB16, W>(A, kw[tt][s], nu, ga, a.alpha, hc, pm);
        __asm__ volatile("" : "+v"(lg[tt][s]));
      }
    float mz = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int64_t t = tbeg + (wv + 4 * tt) * 64 + 16 * s + col;
        const float z = t < T ? a.scale * lg[tt][s] : -INFINITY;
        L.zt[tt * 64 + 16 * s + col][grp] = z;
        mz = fmaxf(mz, z);
        if (a.logits && head < a.qpg && t < T) a.logits[(kg * a.qpg + head) * T + t] = lg[tt][s];
      }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int b = 0; b < VR / 2; ++b)
        if (b * 64 + lane < vunits) reinterpret_cast<u32x4 *>(L.vrec)[tt * vunits + b * 64 + lane] = vr[tt * (VR / 2) + b];
    const float vnl0 = vn[0], vnl1 = vn[1];
    const bool v0 = tbeg + wv * 64 + lane < T, v1 = tbeg + (wv + 4) * 64 + lane < T;
    if (c + 1 < c_end) issue(c + 1);
    wave_sync();

    // ---- B: the wave's running max per head (row grp of every lane holds
    // head grp), rescale factors; plane words of the staged value records;
    // fixed-point weights
    mz = row_max(mz);
    float f[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float mc = lane_f(mz, 16 * h);
      const float mn = fmaxf(M[h], mc);
      f[h] = M[h] == -INFINITY ? 0.f : __expf(M[h] - mn);
      M[h] = mn;
      lsum[h] *= f[h];
    }
    // weights w = exp(z - M) nu <= numax, in units of numax / 127: u = w S,
    // S = 127 / numax, so u <= 127.  The A operand carries u 2^-j (the B byte
    // of bit j of a plane word is 2^j) as four base-128 digits: the bits of
    // U = u 2^(21 - j), an integer below 2^28.
    const float numax = wave_max(fmaxf(v0 ? vnl0 : 0.f, v1 ? vnl1 : 0.f));
    const float S = numax > 0.f ? 127.f / numax : 1.f;
    {
      // lane (record dword k, 32-token block beta) transposes dword k of 32
      // tokens.  Word i is read from token (i + 3 beta) mod 32 (so that the
      // lanes spread over the LDS banks) and the transposed words are rotated
      // back.
      const int ntr = nd * (WT / 32);
      if (lane < ntr) {
        const int k = lane % nd, beta = lane / nd, rot = (3 * beta) & 31;
        uint32_t x[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) x[i] = L.vrec[(32 * beta + ((i + rot) & 31)) * nd + k];
        transpose32(x);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          u32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = __builtin_amdgcn_alignbit(x[4 * i + e], x[4 * i + e], (32 - rot) & 31);
          *reinterpret_cast<u32x4 *>(&L.tpl[beta * TSTR + plane_index(32 * k + 4 * i)]) = v;
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int t = tt * 64 + lane;
      const float4 z4 = *reinterpret_cast<const float4 *>(&L.zt[t][0]);
      const float zz[4] = {z4.x, z4.y, z4.z, z4.w};
      const float sc = (tt ? vnl1 : vnl0) * S * __builtin_amdgcn_ldexpf(1.f, 21 - (lane & 7));
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        // 0 for masked tokens (z = -inf; M is -inf too while none of the
        // wave's tokens has been real)
        const float pz = zz[h] == -INFINITY ? 0.f : __expf(zz[h] - M[h]);
        lsum[h] += pz;
        L.ufix[h * UST + uidx(t)] = (uint32_t)rintf(pz * sc);
      }
    }
    wave_sync();

    // ---- C: the value sum of the wave's 128 tokens on int8 MFMA
    {
      const float fg = grp == 0 ? f[0] : grp == 1 ? f[1] : grp == 2 ? f[2] : f[3];
      const float invS = 1.f / S;
      i32x4 Aw[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int tb = tt * 64 + 32 * (grp >> 1) + 4 * (grp & 1);
        uint32_t dw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const u32x4 u = *reinterpret_cast<const u32x4 *>(&L.ufix[ah * UST + uidx(tb + 8 * b)]);
#pragma unroll
          for (int e = 0; e < 4; ++e) dw[e] |= __builtin_amdgcn_ubfe(u[e], ash, 7) << (8 * b);
        }
        // bytes of bit 7 (dword 3 of the odd lane groups) negated bytewise
        if (grp & 1) dw[3] = (0x80808080u - dw[3]) ^ 0x80808080u;
        Aw[tt] = i32x4{(int)dw[0], (int)dw[1], (int)dw[2], (int)dw[3]};
      }
      // W = sum of the weights (all-ones B), the offset of every plane, as
      // digit pairs; K = sum of the plane coefficients
      const i32x4 ones = vplanes(0xffffffffu);
      i32x4 accW = mfma8(Aw[0], ones, i32x4{0, 0, 0, 0});
      accW = mfma8(Aw[1], ones, accW);
      float K = 0.f;
#pragma unroll
      for (int pl = 0; pl < NPL; ++pl) K += a.vbasis[pl];
      const float KWh = K * (float)(accW[0] * 128 + accW[1]), KWl = K * (float)(accW[2] * 128 + accW[3]);
      const uint32_t *tw0 = &L.tpl[(grp >> 1) * TSTR];
      const uint32_t *tw1 = &L.tpl[(2 + (grp >> 1)) * TSTR];
      // fixed trip count (the tiles past d are skipped) so that the MFMAs of
      // one tile overlap the recombination of the previous one
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        if (ct >= nct) break;
        // bit rows of coordinate 16 ct + col.  Rows past the record hold no
        // bit of a real coordinate: they only reach coordinates >= d, whose
        // sums are never used, and lie inside the row (16 nct VW <= NPMAX)
        int pr[VW];
#pragma unroll
        for (int p = 0; p < VW; ++p) pr[p] = pr0[p] + (16 * VW + 4) * ct;
        i32x4 pacc[NPL];
#pragma unroll
        for (int pl = 0; pl < NPL; ++pl) pacc[pl] = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const uint32_t *tw = tt ? tw1 : tw0;
          uint32_t pw[VW];
#pragma unroll
          for (int p = 0; p < VW; ++p) pw[p] = tw[pr[p]];
#pragma unroll
          for (int p = 0; p < VW; ++p) pacc[p] = mfma8(Aw[tt], vplanes(pw[p]), pacc[p]);
          if constexpr (VW == 3) {
            pacc[3] = mfma8(Aw[tt], vplanes(pw[0] ^ pw[1] ^ pw[2]), pacc[3]);
          } else if constexpr (VW == 4) {
            pacc[4] = mfma8(Aw[tt], vplanes(pw[0] ^ pw[1] ^ pw[2]), pacc[4]);
            pacc[5] = mfma8(Aw[tt], vplanes(pw[0] ^ pw[1] ^ pw[3]), pacc[5]);
            pacc[6] = mfma8(Aw[tt], vplanes(pw[0] ^ pw[2] ^ pw[3]), pacc[6]);
            pacc[7] = mfma8(Aw[tt], vplanes(pw[1] ^ pw[2] ^ pw[3]), pacc[7]);
          }
        }
        // sum_P A_P (2 V_P - W): digit pairs (d0 * 128 + d1, d2 * 128 + d3) of
        // every plane are exact in int32 and in fp32 (below 2^23)
        float sh = 0.f, sl = 0.f;
#pragma unroll
        for (int pl = 0; pl < NPL; ++pl) {
          sh = fmaf(a.vbasis[pl], (float)(pacc[pl][0] * 128 + pacc[pl][1]), sh);
          sl = fmaf(a.vbasis[pl], (float)(pacc[pl][2] * 128 + pacc[pl][3]), sl);
        }
        const float v = fmaf(fmaf(2.f, sl, -KWl), 0x1.0p-21f, fmaf(2.f, sh, -KWh) * 0x1.0p-7f);
        vac[16 * ct] = fmaf(v, invS, vac[16 * ct] * fg);
      }
    }
    wave_sync();          // the wave's zt, vrec, tpl and ufix are rewritten for its next tokens
  }

  // ---- D: merge the four waves' softmax states: every wave's sums are
  // rescaled to the block max of each head
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const float t = wave_sum(lsum[h]);
    if (lane == 0) {
      fin[wv][h][0] = M[h];
      fin[wv][h][1] = t;
    }
  }
  __syncthreads();
  float *out = a.part + (gidx * a.nsplit + blockIdx.x) * 4 * (d + 2);
  for (int i = tid; i < 4 * d; i += NT) {
    const int h = i / d, cc = i - h * d;
    float mb = fin[0][h][0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) mb = fmaxf(mb, fin[w][h][0]);
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
      const float mw = fin[w][h][0];
      v += mw == -INFINITY ? 0.f : wl[w].vacc[h][cc] * __expf(mw - mb);
    }
    out[h * (d + 2) + cc] = v;
  }
  if (tid < 4) {
    const int h = tid;
    float mb = fin[0][h][0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) mb = fmaxf(mb, fin[w][h][0]);
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
      const float mw = fin[w][h][0];
      l += mw == -INFINITY ? 0.f : fin[w][h][1] * __expf(mw - mb);
    }
    out[h * (d + 2) + d] = mb;
    out[h * (d + 2) + d + 1] = l;
  }
}

struct CombArgs {
  const float *part;
  const float *Piv;         // value rotation, row-major [d][d]
  float *out;               // [G][qpg][d]
  float *mstat;             // [G][qpg][2] (max, sum) for the probs pass
  int64_t G;
  int qpg, hg, nchunk, d;
};

// One block per (group, head): chunk weights exp(m_c - M) in LDS, then 1024
// threads = (1024 / d) chunk lanes x d coordinates sum the rescaled partials.
constexpr int CT = 1024;
constexpr int MAXCH_LDS = 8192;     // chunk weights held in LDS (T <= 4M tokens)

__global__ void __launch_bounds__(CT) attend_combine_kernel(CombArgs a) {
  __shared__ float y[TQ_MAX_D];
  __shared__ float wts[MAXCH_LDS];
  __shared__ float red[CT / 64];
  __shared__ float part_acc[CT];
  const int tid = threadIdx.x;
  const int64_t gq = blockIdx.x;             // (group, head)
  const int64_t kg = gq / a.qpg;
  const int h = (int)(gq - kg * a.qpg);
  const int hgi = h / 4, hh = h % 4;
  const int d = a.d;
  const int64_t cstride = 4 * (d + 2);
  const float *p = a.part + ((kg * a.hg + hgi) * a.nchunk) * cstride + hh * (d + 2);
  // global max over chunks
  float m = -INFINITY;
  for (int c = tid; c < a.nchunk; c += CT) m = fmaxf(m, p[c * cstride + d]);
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  float M = red[0];
  for (int i = 1; i < CT / 64; ++i) M = fmaxf(M, red[i]);
  __syncthreads();
  // chunk weights and the total
  float l = 0.f;
  for (int c = tid; c < a.nchunk; c += CT) {
    const float wc = __expf(p[c * cstride + d] - M);
    wts[c] = wc;
    l += p[c * cstride + d + 1] * wc;
  }
  for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
  if ((tid & 63) == 0) red[tid >> 6] = l;
  __syncthreads();
  float L = 0.f;
  for (int i = 0; i < CT / 64; ++i) L += red[i];
  // rescaled sum of the partial vectors
  const int lanes_c = CT / d;                // chunk lanes
  const int ci = tid / d, i = tid - ci * d;
  float v = 0.f;
  if (ci < lanes_c) {
#pragma unroll 4
    for (int c = ci; c < a.nchunk; c += lanes_c) v = fmaf(p[c * cstride + i], wts[c], v);
  }
  part_acc[tid] = v;
  __syncthreads();
  if (tid < d) {
    float s = 0.f;
    for (int k = 0; k < lanes_c; ++k) s += part_acc[k * d + tid];
    y[tid] = s / L;
  }
  __syncthreads();
  for (int jx = tid; jx < d; jx += CT) {      // out = Pi_v^T y
    float o = 0.f;
#pragma unroll 8
    for (int r = 0; r < d; ++r) o = fmaf(a.Piv[(int64_t)r * d + jx], y[r], o);
    a.out[gq * d + jx] = o;
  }
  if (a.mstat && tid == 0) {
    a.mstat[2 * gq] = M;
    a.mstat[2 * gq + 1] = L;
  }
}

__global__ void __launch_bounds__(256) attend_probs_kernel(const float *logits, const float *mstat,
                                                          float *probs, int64_t T, float scale) {
  const int64_t row = blockIdx.y;
  const float M = mstat[2 * row], invL = 1.f / mstat[2 * row + 1];
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < T; t += (int64_t)gridDim.x * 256)
    probs[row * T + t] = __expf(scale * logits[row * T + t] - M) * invL;
}

// Key geometries d <= 128 produces (one sign word per lane group) x value
// code widths 1..4.
int dispatch(const AttArgs &a, dim3 grid, int cb16, int sb16, int w, int vw, hipStream_t s) {
#define TQ_CASE_V(C, S, W_, V)                                         \
  if (vw == V) {                                                       \
    attend_partial_kernel<C, S, W_, V><<<grid, NT, 0, s>>>(a);         \
    return hip_status();                                               \
  }
#define TQ_CASE(C, S, W_)                                              \
  if (cb16 == C && sb16 == S && w == W_) {                             \
    TQ_CASE_V(C, S, W_, 1) TQ_CASE_V(C, S, W_, 2) TQ_CASE_V(C, S, W_, 3) TQ_CASE_V(C, S, W_, 4) \
    return TQ_ENOTSUP;                                                 \
  }
  TQ_CASE(1, 1, 1) TQ_CASE(1, 1, 2) TQ_CASE(2, 1, 2) TQ_CASE(1, 1, 3) TQ_CASE(2, 1, 3) TQ_CASE(3, 1, 3)
#undef TQ_CASE
#undef TQ_CASE_V
  return TQ_ENOTSUP;
}

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// ------------------------------------------------------------ d > 128
// Vectors longer than 128 coordinates take three steps: the logits by the
// scores kernels (into the logits output, or the workspace), a value-sum
// kernel that reads them back with the same online softmax per run of chunks
// and accumulates sum_t exp(z_t - M) nu_t c_v[idx_t] on the VALU, and the
// combine (and probs) kernels above.  Block = (query group of 4 heads, run of
// chunks); thread = (token lane, 4 consecutive coordinates), so that the
// codes of its coordinates are one bit field of a record word pair.
constexpr int VT = 64;             // tokens per value tile

struct VsumArgs {
  const float *logits;             // [G][qpg][T]
  const uint8_t *vcodes;
  const float *vnorms;
  float *part;                     // [G*hg][nsplit][4][d + 2]
  int64_t T, ldk;
  int qpg, hg, cps, nsplit, d, vw, vcb;
  float scale;
  float cf[16];                    // value centroids
};

__global__ void __launch_bounds__(256) attend_vsum_kernel(VsumArgs a) {
  extern __shared__ __align__(16) uint32_t vrec[];   // [VT][vcb / 4] the tile's value records
  __shared__ float4 wt[VT];                          // per token: exp(z - M) nu for the 4 heads
  __shared__ float cbk[16];
  __shared__ float fsc[4];
  __shared__ float4 red[256 * 4];                    // per thread: 4 coordinates x 4 heads
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t gy = blockIdx.y;                     // key group * hg + head group
  const int64_t kg = gy / a.hg;
  const int hgi = (int)(gy - kg * a.hg);
  const int d = a.d, vw = a.vw, vcw = a.vcb / 4;
  const int nq4 = d / 4, nl = 256 / nq4;             // coordinate quads, token lanes
  const int qi = tid % nq4, tl = tid / nq4;
  const bool act = tl < nl;
  if (tid < 16) cbk[tid] = a.cf[tid];
  const int head = hgi * 4 + wv;                     // wave wv keeps head wv's softmax state
  const bool hok = head < a.qpg;
  const float *lrow = a.logits + (kg * a.qpg + (hok ? head : 0)) * a.T;
  const uint8_t *vbase = a.vcodes + kg * a.ldk * a.vcb;
  const float *nbase = a.vnorms + kg * a.ldk;
  float M = -INFINITY, S = 0.f;
  float4 acc[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = make_float4(0.f, 0.f, 0.f, 0.f);
  const int64_t t_begin = (int64_t)blockIdx.x * a.cps * CH;
  const int64_t t_end = min(t_begin + (int64_t)a.cps * CH, a.T);
  const uint32_t cmask = (1u << vw) - 1u;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += VT) {
    const int ntok = (int)min((int64_t)VT, t_end - t0);
    for (int i = tid; i < VT * vcw; i += 256) {
      const int tok = i / vcw;
      vrec[i] = tok < ntok ? reinterpret_cast<const uint32_t *>(vbase + (t0 + tok) * a.vcb)[i - tok * vcw] : 0u;
    }
    const bool tv = hok && lane < ntok;
    const float z = tv ? a.scale * lrow[t0 + lane] : -INFINITY;
    const float Mn = fmaxf(M, wave_max(z));
    const float f = M == -INFINITY ? 0.f : __expf(M - Mn);
    const float pz = z == -INFINITY ? 0.f : __expf(z - Mn);
    S = fmaf(S, f, wave_sum(pz));
    M = Mn;
    const float nu = lane < ntok ? nbase[t0 + lane] : 0.f;
    reinterpret_cast<float *>(&wt[lane])[wv] = pz * nu;
    if (lane == 0) fsc[wv] = f;
    __syncthreads();
    const float4 fs = make_float4(fsc[0], fsc[1], fsc[2], fsc[3]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e].x *= fs.x;
      acc[e].y *= fs.y;
      acc[e].z *= fs.z;
      acc[e].w *= fs.w;
    }
    if (act) {
      const int bit = 4 * qi * vw, wi = bit >> 5, sh = bit & 31;
      for (int tok = tl; tok < ntok; tok += nl) {
        const float4 w4 = wt[tok];
        const uint32_t *rw = vrec + tok * vcw;
        uint32_t bits = rw[wi] >> sh;
        // the field's bits lie inside the record, so word wi + 1 exists here
        if (sh + 4 * vw > 32) bits |= rw[wi + 1] << (32 - sh);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float c = cbk[(bits >> (e * vw)) & cmask];
          acc[e].x = fmaf(c, w4.x, acc[e].x);
          acc[e].y = fmaf(c, w4.y, acc[e].y);
          acc[e].z = fmaf(c, w4.z, acc[e].z);
          acc[e].w = fmaf(c, w4.w, acc[e].w);
        }
      }
    }
    __syncthreads();
  }
  // token lanes summed in a fixed order; partials out
#pragma unroll
  for (int e = 0; e < 4; ++e) red[tid * 4 + e] = acc[e];
  __syncthreads();
  float *pp = a.part + (gy * a.nsplit + blockIdx.x) * (int64_t)(4 * (d + 2));
  if (act && tl == 0) {
    for (int l = 1; l < nl; ++l)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float4 v = red[(l * nq4 + qi) * 4 + e];
        acc[e].x += v.x;
        acc[e].y += v.y;
        acc[e].z += v.z;
        acc[e].w += v.w;
      }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * qi + e;
      pp[0 * (d + 2) + i] = acc[e].x;
      pp[1 * (d + 2) + i] = acc[e].y;
      pp[2 * (d + 2) + i] = acc[e].z;
      pp[3 * (d + 2) + i] = acc[e].w;
    }
  }
  if (lane == 0) {
    pp[wv * (d + 2) + d] = M;
    pp[wv * (d + 2) + d + 1] = S;
  }
}

}  // namespace

size_t attend_ws_bytes(const tq_ctx *k, int64_t G, int qpg, int64_t T) {
  const int hg = (qpg + 3) / 4;
  const int nm = mfma_count(k->cw16, k->sign_bytes / 16, k->hp.w);
  const int64_t nchunk = (T + CH - 1) / CH;
  const int d = k->hp.d;
  // d > 128: the logits of the three-step path as well
  const int64_t lg = d > 128 ? align256(G * qpg * T * 4) : 0;
  return (size_t)(align256(G * hg * prep_stride(nm)) + align256(G * hg * nchunk * 4 * (d + 2) * 4) +
                  align256(G * qpg * 2 * 4) + lg);
}

int check_attend(const tq_ctx *kc, const tq_ctx *vc, int64_t G, int qpg, int64_t T, int64_t ldk,
                 bool want_probs) {
  const int d = kc->hp.d;
  if (vc->hp.w < 1 || vc->hp.w > 4) return TQ_ENOTSUP;
  // the fused kernel (d <= 128) holds a value record in 16 w bytes
  if (d <= 128 && vc->code_bytes > 16 * vc->hp.w) return TQ_ENOTSUP;
  const int64_t groups = G * ((qpg + 3) / 4);
  if (groups > 65535 || T > 0x7fffffff - CH || G * qpg > 0x7fffffff) return TQ_ENOTSUP;
  const int64_t rec_max = std::max<int64_t>(std::max(kc->code_bytes, kc->sign_bytes), vc->code_bytes);
  if (ldk * rec_max >= ((int64_t)1 << 32)) return TQ_ENOTSUP;
  if (want_probs && G * qpg > 65535) return TQ_ENOTSUP;   // probs pass: one grid row per (group, head)
  return TQ_OK;
}

int launch_attend(const tq_ctx *kc, const tq_ctx *vc, const float *q, int64_t G, int qpg, int64_t T,
                  int64_t ldk, const uint8_t *kcodes, const uint8_t *ksigns, const float *knorms,
                  const float *krnorms, const uint8_t *vcodes, const float *vnorms, float scale,
                  float *logits, float *probs, float *out, void *ws, hipStream_t stream,
                  bool prepped) {
  const int d = kc->hp.d;
  if (probs && !logits) return TQ_EINVAL;
  int st = check_attend(kc, vc, G, qpg, T, ldk, probs != nullptr);
  if (st != TQ_OK) return st;
  const int hg = (qpg + 3) / 4;
  const int cb16 = kc->cw16, sb16 = kc->sign_bytes / 16, w = kc->hp.w;
  const int nm = mfma_count(cb16, sb16, w);
  const int64_t nchunk = (T + CH - 1) / CH;
  const int64_t groups = G * hg;
  uint8_t *base = reinterpret_cast<uint8_t *>(ws);
  uint8_t *prep = base;
  float *part = reinterpret_cast<float *>(base + align256(groups * prep_stride(nm)));
  float *mstat = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(part) +
                                           align256(groups * nchunk * 4 * (d + 2) * 4));
  if (!prepped) {                      // else the queries are already prepared in ws
    st = launch_prep(kc, q, groups, qpg, hg, G * qpg, prep, stream);
    if (st != TQ_OK) return st;
  }
  // splits per query group: about TQ_ATT_BLOCKS blocks in all, equal runs of chunks
  int64_t want = (TQ_ATT_BLOCKS + groups - 1) / groups;
  if (want > nchunk) want = nchunk;
  if (want < 1) want = 1;
  const int cps = (int)((nchunk + want - 1) / want);
  const int nsplit = (int)((nchunk + cps - 1) / cps);
  if (d > 128) {
    float *lg = logits ? logits
                       : reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(mstat) + align256(G * qpg * 2 * 4));
    st = launch_scores_prepared(kc, prep, G, qpg, T, ldk, kcodes, ksigns, knorms, krnorms, lg, stream);
    if (st != TQ_OK) return st;
    VsumArgs v{};
    v.logits = lg;
    v.vcodes = vcodes;
    v.vnorms = vnorms;
    v.part = part;
    v.T = T;
    v.ldk = ldk;
    v.qpg = qpg;
    v.hg = hg;
    v.cps = cps;
    v.nsplit = nsplit;
    v.d = d;
    v.vw = vc->hp.w;
    v.vcb = vc->code_bytes;
    v.scale = scale;
    for (int i = 0; i < 16; ++i) v.cf[i] = vc->cf[i];
    attend_vsum_kernel<<<dim3((unsigned)nsplit, (unsigned)groups), 256, (size_t)VT * vc->code_bytes, stream>>>(v);
    if (hip_status() != TQ_OK) return TQ_EHIP;
  } else {
  AttArgs a{};
  a.kcodes = kcodes;
  a.ksigns = ksigns;
  a.knorms = knorms;
  a.krnorms = krnorms;
  a.vcodes = vcodes;
  a.vnorms = vnorms;
  a.prep = prep;
  a.logits = logits;
  a.part = part;
  a.T = T;
  a.ldk = ldk;
  a.qpg = qpg;
  a.hg = hg;
  a.nchunk = (int)nchunk;
  a.cps = cps;
  a.nsplit = nsplit;
  a.d = d;
  a.kcb = kc->code_bytes;
  a.ksb = kc->sign_bytes;
  a.vcb = vc->code_bytes;
  a.alpha = kc->alpha;
  a.scale = scale;
  for (int i = 0; i < 8; ++i) a.vbasis[i] = vc->vbasis[i];
  st = dispatch(a, dim3((unsigned)a.nsplit, (unsigned)groups), cb16, sb16, w, vc->hp.w, stream);
  if (st != TQ_OK) return st;
  }
  CombArgs c{};
  c.part = part;
  c.Piv = vc->Pi32;
  c.out = out;
  c.mstat = probs ? mstat : nullptr;
  c.G = G;
  c.qpg = qpg;
  c.hg = hg;
  c.nchunk = nsplit;
  c.d = d;
  attend_combine_kernel<<<(unsigned)(G * qpg), CT, 0, stream>>>(c);
  if (hip_status() != TQ_OK) return TQ_EHIP;
  if (probs) {
    const int64_t rows = G * qpg;       // <= 65535 (check_attend)
    const unsigned gx = (unsigned)((T + 256 * 8 - 1) / (256 * 8));
    attend_probs_kernel<<<dim3(gx, (unsigned)rows), 256, 0, stream>>>(logits, mstat, probs, T, scale);
    return hip_status();
  }
  return TQ_OK;
}

}  // namespace tq
