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
//        output); the chunk's value records are already on their way into
//        LDS (copied by the memory system, issued one chunk ahead);
//     B. chunk max, running max M, rescale factor f = exp(M_old - M_new);
//        weights w_t = exp(z_t - M) nu_t turned into int8 fixed-point digits
//        (the A operand of the value sum);
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
// chunk), the B operand one byte per token whose bit j is that token's plane
// bit of coordinate 8 n + j (n = the operand column).  Value records store
// their codes as bit planes (one byte = 8 coordinates of one plane), so the
// B operand of a 16-lane group is a byte transpose of 16 records, which the
// LDS does in hardware (ds_read_b64_tr_b8: lane 2r + h names row r, bytes
// 8h .. 8h+7, of an 8 x 16 byte tile; lane i receives column i of the 8 rows,
// row r in byte r).  Masking the bytes with 0x01010101 << j selects
// coordinate 8 n + j (byte value 2^j, -128 for j = 7, undone after the
// product); the parity planes are XORs of plane bytes.  W is the same product
// against all-ones bytes, so 2 V - W is exact in int32 before the digits are
// recombined in fp32.
#include <algorithm>
#include <cfloat>

#include "tq_score_core.h"

namespace tq {
namespace {

constexpr int CH = 512;            // tokens per chunk
constexpr int NT = 256;            // threads per partial block
#ifndef TQ_ATT_BLOCKS
#define TQ_ATT_BLOCKS 512          // partial blocks per call (2 per CU are resident)
#endif

// odd monomials of the code bits of a w-bit value code: w singles + triples
__host__ __device__ constexpr int value_planes(int vw) { return vw + (vw == 3 ? 1 : vw == 4 ? 4 : 0); }

// the fused kernel: d = 64 or 128 (a value plane is one or two 8-byte rows
// of the LDS transpose read)
bool attend_fused(int d) { return d == 64 || d == 128; }

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

typedef int i32x2 __attribute__((ext_vector_type(2)));
// LDS transpose read of 8-bit elements (see the header comment)
__device__ __forceinline__ i32x2 lds_tr8(const uint8_t *p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2 *)(p));
}

// Raw buffer resource over `bytes` bytes from `base`: reads at or beyond
// `bytes` return zero instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
// One non-temporal 32-bit read at byte offset off + imm (imm a constant,
// which the instruction carries).
__device__ __forceinline__ uint32_t buf_word(__amdgpu_buffer_rsrc_t r, uint32_t off, int imm) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)(off + (uint32_t)imm), 0, 2 /* nt */);
}
// 1 KB units I .. N-1 (16 bytes per lane, lane offset included in vo) from
// byte offset vo + 1024 I into LDS at dst + 1024 I, non-temporal.  The
// instruction's constant offset moves the source and the LDS destination
// alike; it stays below 4 KB, so every fourth unit advances both bases.
template <int I, int N>
__device__ __forceinline__ void buf_copy_lds(__amdgpu_buffer_rsrc_t r, uint8_t *dst, uint32_t vo) {
  if constexpr (I < N) {
    constexpr int HI = (I >> 2) * 4096, LO = (I & 3) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(dst + HI), 16,
                                             (int)(vo + (uint32_t)HI), 0, LO, 2 /* nt */);
    buf_copy_lds<I + 1, N>(r, dst, vo);
  }
}

// One block = one query group x one split (a run of `cps` chunks of CH
// tokens).  Wave wv owns the 64-token blocks wv and wv + 4 of every chunk and
// everything computed from them: their logits, staged value records,
// fixed-point weights and value sums, with an online softmax of its own
// (running max M and sum of exp per head; the value sums are rescaled by
// exp(M_old - M_new) whenever its tokens raise the max).  The waves therefore
// never wait for each other inside the chunk loop; their four partial softmax
// states are merged once at the end.  The key words and norms of the wave's
// next tokens are loaded into registers while the current ones are scored,
// and the next value records are copied into the wave's LDS slot by the
// memory system (buffer loads into LDS, 16 bytes per lane) during the next logits.
#ifndef TQ_ATT_WAVES_PER_EU
#define TQ_ATT_WAVES_PER_EU 2
#endif
template <int D, int CB16, int SB16, int W, int VW>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(TQ_ATT_WAVES_PER_EU)))
attend_partial_kernel(AttArgs a) {
  constexpr int NM = ScoreShape<CB16, SB16, W>::NM;
  using KW = KeyWords<CB16, SB16, W>;
  constexpr int NPL = value_planes(VW);
  constexpr int PB = D / 8;                       // bytes per value bit plane
  constexpr int VCB = (VW * PB + 15) / 16 * 16;   // value record bytes
  constexpr int NU16 = VCB / 16;                  // 1 KB copies per 64-token block
  constexpr int WT = 128;                         // tokens of a wave per chunk
  // fixed-point weights U = w S 2^21, [head][token] with a skew of 4 words
  // per 32 tokens
  constexpr int UST = WT + WT / 8 + 4;
  auto uidx = [](int t) { return t + 4 * (t >> 5); };
  // value record slots: token-major (+ the 8 bytes a d = 64 row read
  // passes); two per wave where two blocks of 4 waves still fit a CU's LDS
  // (the next chunk's records are then copied while this chunk is scored),
  // else one (refilled after the value sum)
  constexpr int SLOT = WT * VCB + 16;
  constexpr bool DB = 2 * (4 * (2048 + 2 * SLOT + 16 * UST) + 128) <= 160 * 1024;
  constexpr int NSLOT = DB ? 2 : 1;
  struct WaveLds {
    float zt[WT][4];                              // scaled logits [token][head]
    uint32_t ufix[4 * UST];                       // fixed-point weights
    union __align__(16) {
      uint8_t vrec[NSLOT][SLOT];                  // value records
      float vacc[4][128 + 16];                    // at the end: value sums [head][rotated coordinate]
    };
  };
  __shared__ __align__(16) WaveLds wl[NT / 64];
  __shared__ float fin[NT / 64][4][2];            // per wave and head: running max, sum of exp

  const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, grp = lane >> 4;
  // wave index as a scalar: the wave's LDS and token offsets are then
  // scalar arithmetic
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  WaveLds &L = wl[wv];
  const int64_t gidx = blockIdx.y, kg = gidx / a.hg;
  const int hgi = (int)(gidx - kg * a.hg);
  const int c_begin = blockIdx.x * a.cps;
  const int c_end = min(c_begin + a.cps, a.nchunk);
  constexpr int d = D;
  const int64_t T = a.T;

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
  const uint8_t *vcbp = a.vcodes + kg * a.ldk * VCB;
  const float *vnb = a.vnorms + kg * a.ldk;
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

  // registers of the wave's tokens in flight: key words per 16-key subtile,
  // key norms one per lane (handed out by cross-lane reads) and the value
  // norms of tokens lane and lane + 64
  KW kw[2][4];
  float knu[2], kga[2], vn[2];
  // The group's records are read through buffer resources whose size is the
  // T records of the group: reads past the cache end (the last, partial
  // chunk) return zeros instead of faulting, so no token index is clamped;
  // those tokens get logit -inf and weight 0.  Offsets are 32-bit (the host
  // checks that a group's records span less than 4 GB): one lane offset per
  // 64-token block, the subtile and word offsets immediate.
  const uint32_t Tu = (uint32_t)T;
  const __amdgpu_buffer_rsrc_t rkc = buf_rsrc(kcb, Tu * (CB16 * 16)), rks = buf_rsrc(ksb, Tu * (SB16 * 16));
  const __amdgpu_buffer_rsrc_t rkn = buf_rsrc(knb, Tu * 4), rkr = buf_rsrc(krb, Tu * 4);
  const __amdgpu_buffer_rsrc_t rvc = buf_rsrc(vcbp, Tu * VCB), rvn = buf_rsrc(vnb, Tu * 4);
  // lane offsets within a 64-token block: key words of token col, lane
  // group grp
  const uint32_t kco = (uint32_t)col * (CB16 * 16) + (uint32_t)grp * (CB16 * 4);
  const uint32_t kso = (uint32_t)col * (SB16 * 16) + (uint32_t)grp * (SB16 * 4);
  auto issue = [&](int c) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const uint32_t tb = (uint32_t)(c * CH + (wv + 4 * tt) * 64);   // first token of the block
      uint32_t co = tb * (CB16 * 16) + kco, so = tb * (SB16 * 16) + kso, no = (tb + (uint32_t)lane) * 4;
      // (opaque, so that each load's offset is this value plus an immediate
      // and not a register of its own derived across iterations)
      __asm__ volatile("" : "+v"(co), "+v"(so), "+v"(no));
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int i = 0; i < CB16; ++i) kw[tt][s].cw[i] = buf_word(rkc, co, s * 16 * (CB16 * 16) + 4 * i);
#pragma unroll
        for (int i = 0; i < SB16; ++i) kw[tt][s].sw[i] = buf_word(rks, so, s * 16 * (SB16 * 16) + 4 * i);
      }
      knu[tt] = __uint_as_float(buf_word(rkn, no, 0));
      kga[tt] = __uint_as_float(buf_word(rkr, no, 0));
      vn[tt] = __uint_as_float(buf_word(rvn, no, 0));
    }
  };
  // the value records of the wave's two 64-token blocks of chunk c into its
  // LDS slot: each block is one contiguous run of 64 VCB bytes, moved as
  // 16-byte units by the memory system (units past the cache end arrive as
  // zeros; their tokens get zero weight)
  auto stage_values = [&](int c, int slot) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const uint32_t tb = (uint32_t)(c * CH + (wv + 4 * tt) * 64);
      uint32_t vo = tb * VCB + 16 * (uint32_t)lane;
      __asm__ volatile("" : "+v"(vo));
      uint8_t *dst = L.vrec[slot] + tt * 64 * VCB;
      buf_copy_lds<0, NU16>(rvc, dst, vo);
    }
  };

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
  // value sums of head grp, coordinates 8 col + j (rotated domain)
  float vac[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) vac[j] = 0.f;
  // A operand of the value sum: lane (row m = 4 h + digit, group g) holds, at
  // dword e and byte b, digit (m & 3) of head (m >> 2) for token
  // 16 g + 4 e + b of a 64-token block
  const int ah = col >> 2, ash = 21 - 7 * (col & 3);
  // B operand rows: lane 2r + h of each 16-lane group names bytes 8h .. 8h+7
  // of token 16 grp + r (and 16 grp + 8 + r) in a plane
  const int brow = (16 * grp + (col >> 1)) * VCB + 8 * (col & 1);
  float K = 0.f;
#pragma unroll
  for (int pl = 0; pl < NPL; ++pl) K += a.vbasis[pl];

  issue(c_begin);
  stage_values(c_begin, 0);
  // every load of a chunk (key words, norms, the next chunk's value copies)
  // lands before the chunk is processed: an explicit wait here and at the
  // end of each iteration (the compiler does not order the LDS copies before
  // the slot's reads)
  wait_vm<0>();
  for (int c = c_begin; c < c_end; ++c) {
    const int slot = DB ? (c - c_begin) & 1 : 0;
    // ---- A: logits of the wave's tokens into LDS
    float lg[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const float aga = a.alpha * kga[tt];        // alpha gamma, once per token
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if constexpr (W == 3) {   // first code word of the next lane group (lane + 16), none for the last
          const uint32_t nxt = (uint32_t)__shfl((int)kw[tt][s].cw[0], (lane + 16) & 63);
          kw[tt][s].cw[CB16] = grp < 3 ? nxt : 0u;
        }
        const float nu = __shfl(knu[tt], 16 * s + col), ga = __shfl(aga, 16 * s + col);
        lg[tt][s] = tile_logit<CB16, SB16, W>(A, kw[tt][s], nu, ga, 1.f, hc, pm);
        __asm__ volatile("" : "+v"(lg[tt][s]));
      }
    }
    // (token indexes fit in 32 bits: the host limits T to 2^31 - CH)
    const int Ti = (int)T, tb32 = c * CH;
    float mz = -INFINITY;
    if ((c + 1) * CH <= Ti) {
      // a whole chunk: every token is real
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float z = a.scale * lg[tt][s];
          L.zt[tt * 64 + 16 * s + col][grp] = z;
          mz = fmaxf(mz, z);
          if (a.logits && head < a.qpg)
            a.logits[(kg * a.qpg + head) * T + tb32 + (wv + 4 * tt) * 64 + 16 * s + col] = lg[tt][s];
        }
    } else {
      // the last, partial chunk: tokens past the cache end get -inf
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int t = tb32 + (wv + 4 * tt) * 64 + 16 * s + col;
          const float z = t < Ti ? a.scale * lg[tt][s] : -INFINITY;
          L.zt[tt * 64 + 16 * s + col][grp] = z;
          mz = fmaxf(mz, z);
          if (a.logits && head < a.qpg && t < Ti) a.logits[(kg * a.qpg + head) * T + t] = lg[tt][s];
        }
    }
    const float vnl0 = vn[0], vnl1 = vn[1];
    const bool v0 = tb32 + wv * 64 + lane < Ti, v1 = tb32 + (wv + 4) * 64 + lane < Ti;
    if (c + 1 < c_end) {
      issue(c + 1);
      if constexpr (DB) stage_values(c + 1, slot ^ 1);
    }
    wave_sync();

    // ---- B: the wave's running max per head (row grp of every lane holds
    // head grp), rescale factors; fixed-point weights
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
    // S = 127 / numax, so u <= 127; the A operand carries the four base-128
    // digits of U = u 2^21, an integer below 2^28
    // (S from the hardware reciprocal, 2^-20 below 127 / numax so that u stays
    // below 127 whatever its rounding; S only has to be that bound)
    const float numax = wave_max(fmaxf(v0 ? vnl0 : 0.f, v1 ? vnl1 : 0.f));
    const float S = numax > 0.f ? (127.f * (1.f - 0x1.0p-20f)) * __builtin_amdgcn_rcpf(numax) : 1.f;
    // the running max floored to a finite value: masked tokens (z = -inf)
    // then get exp(-inf) = 0 also while none of the wave's tokens has been
    // real (M = -inf), with no compare
    float Mf[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) Mf[h] = fmaxf(M[h], -FLT_MAX);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int t = tt * 64 + lane;
      const float4 z4 = *reinterpret_cast<const float4 *>(&L.zt[t][0]);
      const float zz[4] = {z4.x, z4.y, z4.z, z4.w};
      const float sc = (tt ? vnl1 : vnl0) * S * 0x1.0p21f;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float pz = __expf(zz[h] - Mf[h]);
        lsum[h] += pz;
        // rounded to the nearest integer (the sum stays below 2^28, and the
        // conversion truncates)
        L.ufix[h * UST + uidx(t)] = (uint32_t)fmaf(pz, sc, 0.5f);
      }
    }
    wave_sync();

    // ---- C: the value sum of the wave's 128 tokens on int8 MFMA
    {
      const float fg = grp == 0 ? f[0] : grp == 1 ? f[1] : grp == 2 ? f[2] : f[3];
      const float invS = __builtin_amdgcn_rcpf(S);
      i32x4 Aw[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int tb = tt * 64 + 16 * grp;
        uint32_t dw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const u32x4 u = *reinterpret_cast<const u32x4 *>(&L.ufix[ah * UST + uidx(tb + 4 * e)]);
          dw[e] = __builtin_amdgcn_ubfe(u[0], ash, 7) | (__builtin_amdgcn_ubfe(u[1], ash, 7) << 8) |
                  (__builtin_amdgcn_ubfe(u[2], ash, 7) << 16) | (__builtin_amdgcn_ubfe(u[3], ash, 7) << 24);
        }
        Aw[tt] = i32x4{(int)dw[0], (int)dw[1], (int)dw[2], (int)dw[3]};
      }
      // W = sum of the weights (all-ones B) as digit pairs
      const i32x4 ones = i32x4{0x01010101, 0x01010101, 0x01010101, 0x01010101};
      i32x4 accW = mfma8(Aw[0], ones, i32x4{0, 0, 0, 0});
      accW = mfma8(Aw[1], ones, accW);
      const float KWh = K * (float)(accW[0] * 128 + accW[1]), KWl = K * (float)(accW[2] * 128 + accW[3]);
      // plane bytes of the lane's octet for its 16 tokens of each block: the
      // single planes by transpose reads, the triples by XOR
      u32x4 pb4[2][NPL];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const uint8_t *r0 = L.vrec[slot] + tt * 64 * VCB + brow;
#pragma unroll
        for (int p = 0; p < VW; ++p) {
          const i32x2 lo = lds_tr8(r0 + p * PB), hi = lds_tr8(r0 + p * PB + 8 * VCB);
          pb4[tt][p] = u32x4{(unsigned)lo[0], (unsigned)lo[1], (unsigned)hi[0], (unsigned)hi[1]};
        }
        if constexpr (VW == 3) {
          pb4[tt][3] = pb4[tt][0] ^ pb4[tt][1] ^ pb4[tt][2];
        } else if constexpr (VW == 4) {
          pb4[tt][4] = pb4[tt][0] ^ pb4[tt][1] ^ pb4[tt][2];
          pb4[tt][5] = pb4[tt][0] ^ pb4[tt][1] ^ pb4[tt][3];
          pb4[tt][6] = pb4[tt][0] ^ pb4[tt][2] ^ pb4[tt][3];
          pb4[tt][7] = pb4[tt][1] ^ pb4[tt][2] ^ pb4[tt][3];
        }
      }
      // coordinate 8 col + j, j = 0..7: the MFMAs of j are issued before the
      // recombination of j - 1 (two accumulator sets), and the scheduler is
      // kept from mixing more iterations (their operands would not fit)
      i32x4 pacc[2][NPL];
      auto products = [&](int j, i32x4 (&acc)[NPL]) {
        const unsigned msk = 0x01010101u << j;
#pragma unroll
        for (int pl = 0; pl < NPL; ++pl) {
          const u32x4 b0 = pb4[0][pl] & msk, b1 = pb4[1][pl] & msk;
          acc[pl] = mfma8(Aw[0], i32x4{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3]}, i32x4{0, 0, 0, 0});
          acc[pl] = mfma8(Aw[1], i32x4{(int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]}, acc[pl]);
        }
      };
      // sum_P A_P (2 V_P - W): digit pairs (d0 * 128 + d1, d2 * 128 + d3) of
      // every plane are exact in int32; the byte value 2^j (-128 for j = 7)
      // is divided out here
      auto recombine = [&](int j, const i32x4 (&acc)[NPL]) {
        float sh = 0.f, sl = 0.f;
#pragma unroll
        for (int pl = 0; pl < NPL; ++pl) {
          sh = fmaf(a.vbasis[pl], (float)(acc[pl][0] * 128 + acc[pl][1]), sh);
          sl = fmaf(a.vbasis[pl], (float)(acc[pl][2] * 128 + acc[pl][3]), sl);
        }
        const float tj = j == 7 ? -0x1.0p-6f : 2.f / (float)(1 << j);   // 2 / byte value
        const float v = fmaf(fmaf(tj, sl, -KWl), 0x1.0p-21f, fmaf(tj, sh, -KWh) * 0x1.0p-7f);
        vac[j] = fmaf(v, invS, vac[j] * fg);
        // (an empty asm keeps the recombination here: unpinned, the compiler
        // defers every recombination past all 64 products, whose results
        // then no longer fit in registers)
        __asm__ volatile("" : "+v"(vac[j]));
      };
      if constexpr (NPL <= 4) {
        products(0, pacc[0]);
#pragma unroll
        for (int j = 1; j < 8; ++j) {
          products(j, pacc[j & 1]);
          recombine(j - 1, pacc[(j - 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);
        }
        recombine(7, pacc[1]);
      } else {          // 4-bit values: one set (two would spill)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          products(j, pacc[0]);
          recombine(j, pacc[0]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);           // lgkmcnt(0): the slot's reads are done
    wave_sync();          // the wave's zt, vrec and ufix are rewritten for its next tokens
    if constexpr (!DB) {
      if (c + 1 < c_end) stage_values(c + 1, 0);
    }
    wait_vm<0>();
  }
  wave_sync();            // the slots' last reads are done: vacc reuses them
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (8 * col + j < d) L.vacc[grp][8 * col + j] = vac[j];

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
  // out = Pi_v^T y: thread (row lane ri, column jx) sums rows ri, ri + nr, ...
  // (short chains of coalesced row reads; d <= TQ_MAX_D = CT), then the row
  // lanes are added
  {
    const int nr = CT / d;
    const int ri = tid / d, jx = tid - ri * d;
    float o = 0.f;
    if (ri < nr) {
#pragma unroll 4
      for (int r = ri; r < d; r += nr) o = fmaf(a.Piv[(int64_t)r * d + jx], y[r], o);
    }
    if (ri < nr) part_acc[tid] = o;             // (its last reads were before the barrier above)
    __syncthreads();
    if (tid < d) {
      float sum = 0.f;
      for (int k = 0; k < nr; ++k) sum += part_acc[k * d + tid];
      a.out[gq * d + tid] = sum;
    }
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

// Key geometries of d = 64 and 128 (one sign word per lane group) x value
// code widths 1..4.
int dispatch(const AttArgs &a, dim3 grid, int cb16, int sb16, int w, int vw, hipStream_t s) {
#define TQ_CASE_V(D_, C, S, W_, V)                                     \
  if (vw == V) {                                                       \
    attend_partial_kernel<D_, C, S, W_, V><<<grid, NT, 0, s>>>(a);     \
    return hip_status();                                               \
  }
#define TQ_CASE(D_, C, S, W_)                                          \
  if (a.d == D_ && cb16 == C && sb16 == S && w == W_) {                \
    TQ_CASE_V(D_, C, S, W_, 1) TQ_CASE_V(D_, C, S, W_, 2) TQ_CASE_V(D_, C, S, W_, 3) TQ_CASE_V(D_, C, S, W_, 4) \
    return TQ_ENOTSUP;                                                 \
  }
  TQ_CASE(64, 1, 1, 1) TQ_CASE(64, 1, 1, 2) TQ_CASE(64, 2, 1, 3)
  TQ_CASE(128, 1, 1, 1) TQ_CASE(128, 2, 1, 2) TQ_CASE(128, 3, 1, 3)
#undef TQ_CASE
#undef TQ_CASE_V
  return TQ_ENOTSUP;
}

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// ------------------------------------------------------------ other d
// Vectors of other lengths than 64 and 128 take three steps: the logits by the
// scores kernels (into the logits output, or the workspace), a value-sum
// kernel that reads them back with the same online softmax per run of chunks
// and accumulates sum_t exp(z_t - M) nu_t c_v[idx_t] on the VALU, and the
// combine (and probs) kernels above.  Block = (query group of 4 heads, run of
// chunks); thread = (token lane, 4 consecutive coordinates), so that each
// bit plane of a value record holds the thread's coordinates as one nibble.
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
      // bit planes: plane pl holds the 4 coordinates' bits as one nibble at
      // record bit pl d + 4 qi (never across a word)
      for (int tok = tl; tok < ntok; tok += nl) {
        const float4 w4 = wt[tok];
        const uint32_t *rw = vrec + tok * vcw;
        uint32_t nib[4];
#pragma unroll
        for (int pl = 0; pl < 4; ++pl) {
          const int bit = pl * d + 4 * qi;
          nib[pl] = pl < vw ? (rw[bit >> 5] >> (bit & 31)) & 0xfu : 0u;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t code = 0;
#pragma unroll
          for (int pl = 0; pl < 4; ++pl) code |= ((nib[pl] >> e) & 1u) << pl;
          const float c = cbk[code];
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
  // the three-step path (d other than 64 and 128): the logits as well
  const int64_t lg = !attend_fused(d) ? align256(G * qpg * T * 4) : 0;
  return (size_t)(align256(G * hg * prep_stride(nm)) + align256(G * hg * nchunk * 4 * (d + 2) * 4) +
                  align256(G * qpg * 2 * 4) + lg);
}

int check_attend(const tq_ctx *kc, const tq_ctx *vc, int64_t G, int qpg, int64_t T, int64_t ldk,
                 bool want_probs) {
  const int d = kc->hp.d;
  if (vc->hp.w < 1 || vc->hp.w > 4) return TQ_ENOTSUP;
  // the fused kernel holds a value record in 16 w bytes
  if (attend_fused(d) && vc->code_bytes > 16 * vc->hp.w) return TQ_ENOTSUP;
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
  if (!attend_fused(d)) {
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
