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
#include <hip/hip_ext.h>

#include <type_traits>

#include "tq_prep_body.h"

namespace tq {
namespace {

#ifndef TQ_SOFTMAX_NT
#define TQ_SOFTMAX_NT 512     // threads per row for rows of up to 32768 values
#endif
#ifndef TQ_SCORES_WAVES
#define TQ_SCORES_WAVES 16384
#endif


template <int JC, bool SPLIT>
__global__ void __launch_bounds__(PREP_THREADS) prep_kernel(PrepArgs a) {
  __shared__ PrepSmem<SPLIT> sm;
  prep_body<JC, SPLIT>(a, sm, blockIdx.x, threadIdx.x, true);
}

struct ScoreArgs {
  const uint8_t *codes, *signs;
  const float *norms, *rnorms;
  float *logits;
  const uint8_t *ws;
  int64_t T, ldk;
  int qpg, hg, hq, tiles_per_wave, cb, sb;   // hq: blocks of NQ head groups per key group
  int wide;                 // T and the logits base allow one 4*spb-byte store per lane
  float alpha;
};

// 16-key subtiles per wave iteration: a 64-key tile fills one LDS slot of the
// double buffer
constexpr int kScoresSPB = 4;

// NQ groups of 4 queries (head groups) per wave: each key tile's bit-plane
// operands are built once for all of them (many queries per key group, e.g.
// every position of a prefill, are bound by that VALU work, not by bytes).
//
// FRAC: fractional-width records (24 to 80 code bytes, the two halves' bit
// planes by quarter); the tile copies into LDS end with a partial 1 KB
// instruction where the tile's bytes are not a multiple of 1 KB.
// LATE (3-bit codes, one head group): a tile's words are read from its LDS
// slot subtile by subtile while it is scored, and the slot is refilled
// afterwards; without the words of four subtiles held in registers the
// kernel fits four waves per SIMD.
template <int CB16, int SB16, int W, int NQ, bool FRAC>
__host__ __device__ constexpr bool scores_late_refill() { return W == 3 && NQ == 1 && !FRAC; }

template <int CB16, int SB16, int W, int NQ, bool FRAC = false>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(scores_late_refill<CB16, SB16, W, NQ, FRAC>() ? 4 : 1)))
scores_kernel(ScoreArgs a) {
  constexpr int NM = ScoreShape<CB16, SB16, W>::NM;
  constexpr int SPB = kScoresSPB, KT = 16 * SPB;
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const int wv = threadIdx.x >> 6;
  const int64_t gy = blockIdx.y;         // key group * hq + block of NQ head groups
  const int64_t kg = gy / a.hq;
  const int hb = (int)(gy - kg * a.hq);

  // with an odd head-group count the last block's second group repeats the
  // first (its logits are computed and not stored)
  i32x4 A[NQ][NM];
  HeadConsts hc[NQ];
  bool head_ok[NQ];
  float *lrow[NQ];
#pragma unroll
  for (int g = 0; g < NQ; ++g) {
    const int hgi = min(hb * NQ + g, a.hg - 1);
    const uint8_t *prep = a.ws + (kg * a.hg + hgi) * prep_stride(NM);
#pragma unroll
    for (int mu = 0; mu < NM; ++mu) A[g][mu] = reinterpret_cast<const i32x4 *>(prep)[mu * 64 + lane];
    hc[g] = HeadConsts::load(reinterpret_cast<const float *>(prep + NM * 1024) + grp * 4);
    const int head = hgi * 4 + grp;
    head_ok[g] = hb * NQ + g < a.hg && head < a.qpg;
    lrow[g] = a.logits + ((int64_t)kg * a.qpg + (head_ok[g] ? head : 0)) * a.T;
  }
  const ParityMasks<CB16, W> pm = parity_masks<CB16, W>(grp);

  const int T = (int)a.T;                  // T < 2^31 is checked on the host
  const int tile0 = (blockIdx.x * 4 + wv) * a.tiles_per_wave;
  // Record strides are compile-time (code_bytes = 16 CB16, sign_bytes = 16 SB16;
  // fractional widths: 8 (CB16 / W) (2 W - 1) code bytes, the two halves'
  // planes) and per-token offsets are 32-bit from per-group base pointers,
  // which keeps address arithmetic to a few shifts per load.
  constexpr int CBY = FRAC ? 8 * (CB16 / W) * (2 * W - 1) : CB16 * 16, SBY = SB16 * 16;
  const uint8_t *cbase = a.codes + (int64_t)kg * a.ldk * CBY;
  const uint8_t *sbase = a.signs + (int64_t)kg * a.ldk * SBY;
  const float *nbase = a.norms + (int64_t)kg * a.ldk;
  const float *rbase = a.rnorms + (int64_t)kg * a.ldk;
  // fractional widths: lane group g's plane words start at word woff of the
  // record; a second-half quarter has fewer (nreal), and its remaining slots
  // repeat a real word (their A coefficients are zero)
  constexpr int WPP = FRAC ? CB16 / W : 1, NLO = FRAC ? (W - 1) * WPP : CB16;
  const int nreal = grp < 2 ? CB16 : NLO;
  const int woff = grp < 2 ? grp * CB16 : 2 * CB16 + (grp - 2) * NLO;

  int ntile = a.tiles_per_wave;
  const int last = (T + KT - 1) / KT;
  if (tile0 + ntile > last) ntile = last - tile0;
  auto load_tile = [&](KeyWords<CB16, SB16, W> (&kw)[SPB], float (&nu)[SPB], float (&ga)[SPB], int t0) {
#pragma unroll
    for (int s = 0; s < SPB; ++s) {
      const uint32_t t = (uint32_t)min(t0 + 16 * s + col, T - 1);
      if constexpr (FRAC) {
        const uint32_t *cw = reinterpret_cast<const uint32_t *>(cbase + t * (uint32_t)CBY) + woff;
#pragma unroll
        for (int i = 0; i < CB16; ++i) kw[s].cw[i] = key_word<true>(cw + min(i, nreal - 1));
        if constexpr (W == 3) kw[s].cw[CB16] = 0u;
        const uint32_t *sw = reinterpret_cast<const uint32_t *>(sbase + t * (uint32_t)SBY + grp * (SB16 * 4));
#pragma unroll
        for (int i = 0; i < SB16; ++i) kw[s].sw[i] = key_word<true>(sw + i);
      } else {
        load_key_words<true>(kw[s], cbase, sbase, t, grp);
      }
      nu[s] = load_f32(nbase, t);
      ga[s] = load_f32(rbase, t);
    }
  };
  auto score_tile = [&](const KeyWords<CB16, SB16, W> (&kw)[SPB], const float (&nu)[SPB], const float (&ga)[SPB],
                        int t0) {
    // the four 16-key logits first, then the guarded stores; materialising l
    // keeps the norm loads from being sunk into the stores' branches
    float l[SPB][NQ];
#pragma unroll
    for (int s = 0; s < SPB; ++s) {
      tile_logits<CB16, SB16, W, NQ, FRAC>(A, kw[s], nu[s], ga[s], a.alpha, hc, pm, l[s]);
#pragma unroll
      for (int g = 0; g < NQ; ++g) __asm__ volatile("" : "+v"(l[s][g]));
    }
#pragma unroll
    for (int g = 0; g < NQ; ++g)
#pragma unroll
      for (int s = 0; s < SPB; ++s) {
        const int t = t0 + 16 * s + col;
        if (head_ok[g] && t < T) lrow[g][t] = l[s][g];      // cached: the softmax reads them next
      }
  };
  // logits of the tile, [head][key] per wave: each lane then stores SPB
  // consecutive keys of its head with one wide store (one store instruction
  // per tile instead of one per 16-key subtile)
  __shared__ __align__(16) float lt[4][NQ][4][KT];
  typedef float fvec __attribute__((ext_vector_type(SPB)));
  // Full tiles (every key below T; only a group's last tile can be partial)
  // are moved to LDS by the memory system itself: a tile's code bytes and
  // its sign bytes are each one contiguous run, so a wave copies them into
  // its own LDS slot with a few global_load_lds_dwordx4 instructions (16 B
  // per lane, 1 KB each, non-temporal: read once) and then reads the MFMA
  // operand words from LDS; the norms come one per lane into registers and
  // are handed out by cross-lane reads.  Counters showed the kernel's time
  // following the number of load instructions per key rather than bytes
  // (the texture address unit was the busiest part), and this form needs
  // the fewest: CB16 + SB16 + 2 per 64 keys, against 16 or more with one
  // load of each record word per lane.
  constexpr int TB = KT * (CBY + SBY);
  __shared__ __align__(16) uint8_t kbA[4][TB];
  __shared__ __align__(16) uint8_t kbB[4][TB];
  // NB bytes (a multiple of 16) from src to dst, 1 KB per instruction; a
  // remainder takes one more instruction on the lanes it needs
  auto dma = [&](uint8_t *dst, const uint8_t *src, auto nb) {
    constexpr int NB = decltype(nb)::value, FULL = NB / 1024, REM = NB % 1024;
#pragma unroll
    for (int i = 0; i < FULL; ++i)
      __builtin_amdgcn_global_load_lds(src + i * 1024 + lane * 16,
                                       (__attribute__((address_space(3))) void *)(dst + i * 1024), 16, 0,
                                       2 /* nt */);
    if constexpr (REM > 0) {
      if (lane * 16 < REM)
        __builtin_amdgcn_global_load_lds(src + FULL * 1024 + lane * 16,
                                         (__attribute__((address_space(3))) void *)(dst + FULL * 1024), 16, 0,
                                         2 /* nt */);
    }
  };
  auto load_dma = [&](uint8_t (&kb)[4][TB], float &nu, float &ga, int t0) {
    dma(kb[wv], cbase + (uint32_t)t0 * CBY, std::integral_constant<int, KT * CBY>{});
    dma(kb[wv] + KT * CBY, sbase + (uint32_t)t0 * SBY, std::integral_constant<int, KT * SBY>{});
    const uint32_t tl = (uint32_t)(t0 + (lane % KT));
    nu = load_f32(nbase, tl);
    ga = load_f32(rbase, tl);
  };
  // the tile's words from LDS into registers (all subtiles), so that the
  // slot can be refilled at once
  auto read_dma = [&](uint8_t (&kb)[4][TB], KeyWords<CB16, SB16, W> (&kw)[SPB]) {
#pragma unroll
    for (int s = 0; s < SPB; ++s) {
      const int k = 16 * s + col;
      const uint8_t *rsg = kb[wv] + KT * CBY + k * SBY + grp * (SB16 * 4);
      if constexpr (FRAC) {
        const uint8_t *rc = kb[wv] + k * CBY + woff * 4;
#pragma unroll
        for (int i = 0; i < CB16; ++i) kw[s].cw[i] = *reinterpret_cast<const uint32_t *>(rc + 4 * min(i, nreal - 1));
        if constexpr (W == 3) kw[s].cw[CB16] = 0u;
      } else {
        const uint8_t *rc = kb[wv] + k * CBY + grp * (CB16 * 4);
#pragma unroll
        for (int i = 0; i < CB16; ++i) kw[s].cw[i] = *reinterpret_cast<const uint32_t *>(rc + 4 * i);
        if constexpr (W == 3) {   // first code word of the next lane group (in LDS after ours), none for the last
          const uint32_t nxt = *reinterpret_cast<const uint32_t *>(rc + 4 * CB16);
          kw[s].cw[CB16] = grp < 3 ? nxt : 0u;
        }
      }
#pragma unroll
      for (int i = 0; i < SB16; ++i) kw[s].sw[i] = *reinterpret_cast<const uint32_t *>(rsg + 4 * i);
    }
  };
  auto score_dma = [&](const KeyWords<CB16, SB16, W> (&kw)[SPB], float nub, float gab, int t0) {
#pragma unroll
    for (int s = 0; s < SPB; ++s) {
      const float nu = __shfl(nub, 16 * s + col), ga = __shfl(gab, 16 * s + col);
      float l[NQ];
      tile_logits<CB16, SB16, W, NQ, FRAC>(A, kw[s], nu, ga, a.alpha, hc, pm, l);
#pragma unroll
      for (int g = 0; g < NQ; ++g) lt[wv][g][grp][16 * s + col] = l[g];
    }
#pragma unroll
    for (int g = 0; g < NQ; ++g) {
      const fvec v = *reinterpret_cast<const fvec *>(&lt[wv][g][grp][SPB * col]);
      float *dst = lrow[g] + (uint32_t)(t0 + SPB * col);
      if (head_ok[g]) {
        if (a.wide) {
          *reinterpret_cast<fvec *>(dst) = v;
        } else {
#pragma unroll
          for (int i = 0; i < SPB; ++i) dst[i] = v[i];
        }
      }
    }
  };
  // LATE: the words of subtile s of a slot, read right before it is scored
  auto score_dma_slot = [&](uint8_t (&kb)[4][TB], float nub, float gab, int t0) {
#pragma unroll
    for (int s = 0; s < SPB; ++s) {
      KeyWords<CB16, SB16, W> kw1;
      const int k = 16 * s + col;
      const uint8_t *rc = kb[wv] + k * CBY + grp * (CB16 * 4);
      const uint8_t *rsg = kb[wv] + KT * CBY + k * SBY + grp * (SB16 * 4);
#pragma unroll
      for (int i = 0; i < CB16; ++i) kw1.cw[i] = *reinterpret_cast<const uint32_t *>(rc + 4 * i);
      if constexpr (W == 3) {
        const uint32_t nxt = *reinterpret_cast<const uint32_t *>(rc + 4 * CB16);
        kw1.cw[CB16] = grp < 3 ? nxt : 0u;
      }
#pragma unroll
      for (int i = 0; i < SB16; ++i) kw1.sw[i] = *reinterpret_cast<const uint32_t *>(rsg + 4 * i);
      const float nu = __shfl(nub, 16 * s + col), ga = __shfl(gab, 16 * s + col);
      float l[NQ];
      tile_logits<CB16, SB16, W, NQ, FRAC>(A, kw1, nu, ga, a.alpha, hc, pm, l);
#pragma unroll
      for (int g = 0; g < NQ; ++g) lt[wv][g][grp][16 * s + col] = l[g];
    }
#pragma unroll
    for (int g = 0; g < NQ; ++g) {
      const fvec v = *reinterpret_cast<const fvec *>(&lt[wv][g][grp][SPB * col]);
      float *dst = lrow[g] + (uint32_t)(t0 + SPB * col);
      if (head_ok[g]) {
        if (a.wide) {
          *reinterpret_cast<fvec *>(dst) = v;
        } else {
#pragma unroll
          for (int i = 0; i < SPB; ++i) dst[i] = v[i];
        }
      }
    }
  };
  if (ntile <= 0) return;
  // first key of this wave's i-th tile
  auto key0 = [&](int i) { return (tile0 + i) * KT; };
  // (fractional widths: a key group whose records do not start on 16 bytes,
  // ldk * code bytes odd in 8-byte units, is read lane by lane throughout)
  const bool dma_ok = !FRAC || ((a.ldk * CBY) & 15) == 0;
  const int nfull = !dma_ok ? 0 : key0(ntile - 1) + KT > T ? ntile - 1 : ntile;
  // two slots, two tiles in flight: a slot is read into registers, refilled
  // with the tile after next, and only then is its tile scored
  float nA, gA, nB, gB;
  KeyWords<CB16, SB16, W> kw[SPB];
  if (nfull > 0) load_dma(kbA, nA, gA, key0(0));
  if (nfull > 1) load_dma(kbB, nB, gB, key0(1));
  // Before a slot is read, its copy has landed: the only loads issued after
  // it are the other slot's copy (NLD instructions) when that was issued.
  constexpr int NLD = (KT * CBY + 1023) / 1024 + (KT * SBY + 1023) / 1024 + 2;
  auto wait_slot = [](bool other_issued) {
    if (other_issued)
      wait_vm<NLD>();
    else
      wait_vm<0>();
  };
  if constexpr (scores_late_refill<CB16, SB16, W, NQ, FRAC>()) {
    for (int it = 0; it < nfull; it += 2) {
      wait_slot(it + 1 < nfull);                  // A(it) landed (B(it+1) was copied after it)
      score_dma_slot(kbA, nA, gA, key0(it));
      __builtin_amdgcn_s_waitcnt(0xc07f);         // lgkmcnt(0): the slot's reads are done
      if (it + 2 < nfull) load_dma(kbA, nA, gA, key0(it + 2));
      if (it + 1 >= nfull) break;
      wait_slot(it + 2 < nfull);                  // B(it+1) landed (A(it+2) was copied after it)
      score_dma_slot(kbB, nB, gB, key0(it + 1));
      __builtin_amdgcn_s_waitcnt(0xc07f);
      if (it + 3 < nfull) load_dma(kbB, nB, gB, key0(it + 3));
    }
  } else
  for (int it = 0; it < nfull; it += 2) {
    wait_slot(it + 1 < nfull);
    read_dma(kbA, kw);
    float nu = nA, ga = gA;
    __builtin_amdgcn_s_waitcnt(0xc07f);           // lgkmcnt(0): the slot's reads are done
    if (it + 2 < nfull) load_dma(kbA, nA, gA, key0(it + 2));
    score_dma(kw, nu, ga, key0(it));
    if (it + 1 >= nfull) break;
    wait_slot(it + 2 < nfull);
    read_dma(kbB, kw);
    nu = nB;
    ga = gB;
    __builtin_amdgcn_s_waitcnt(0xc07f);
    if (it + 3 < nfull) load_dma(kbB, nB, gB, key0(it + 3));
    score_dma(kw, nu, ga, key0(it + 1));
  }
  for (int i = nfull; i < ntile; ++i) {   // the group's last tile (keys clamped, stores guarded)
    KeyWords<CB16, SB16, W> k0[SPB];
    float n0[SPB], g0[SPB];
    load_tile(k0, n0, g0, key0(i));
    score_tile(k0, n0, g0, key0(i));
  }
}

// Two head groups per wave where both groups' operand fragments fit in
// registers beside the rest (up to 12 MFMAs per 16 keys); four where the
// records take at most 6 (codes of 1 or 2 bits at d <= 128): each bit-plane
// operand then serves four MFMAs (8 groups x 8192 queries x 2048 keys, b=3:
// 306 -> 275 us, at two waves per SIMD instead of three).
constexpr int kScoresNQ2MaxNM = 12;
constexpr int kScoresNQ4MaxNM = 6;

// With events, the dispatch itself records them (hipExtLaunchKernel): they
// bracket exactly this kernel's execution.
template <int C, int S, int W_, int NQ, bool FRAC>
int launch_one(const ScoreArgs &a, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (e0 || e1)
    hipExtLaunchKernelGGL(scores_kernel<C, S, W_, NQ, FRAC>, grid, dim3(256), 0, s, e0, e1, 0, a);
  else
    scores_kernel<C, S, W_, NQ, FRAC><<<grid, 256, 0, s>>>(a);
  return hip_status();
}

template <int C, int S, int W_, bool FRAC = false>
int launch_geometry(const ScoreArgs &a, dim3 grid, int nq, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if constexpr (ScoreShape<C, S, W_>::NM <= kScoresNQ4MaxNM && !FRAC) {
    if (nq == 4) return launch_one<C, S, W_, 4, FRAC>(a, grid, s, e0, e1);
  }
  if constexpr (ScoreShape<C, S, W_>::NM <= kScoresNQ2MaxNM) {
    if (nq == 2) return launch_one<C, S, W_, 2, FRAC>(a, grid, s, e0, e1);
  }
  return launch_one<C, S, W_, 1, FRAC>(a, grid, s, e0, e1);
}

// fractional-width geometries (d = 128, 256 at 2.5 and 3.5 bits):
// (first-half plane words per lane group, sign words, first-half code bits)
int dispatch_frac(const ScoreArgs &a, dim3 grid, int cb16, int sb16, int w, int nq, hipStream_t s,
                  hipEvent_t e0, hipEvent_t e1) {
  if (cb16 == 2 && sb16 == 1 && w == 2) return launch_geometry<2, 1, 2, true>(a, grid, nq, s, e0, e1);
  if (cb16 == 3 && sb16 == 1 && w == 3) return launch_geometry<3, 1, 3, true>(a, grid, nq, s, e0, e1);
  if (cb16 == 4 && sb16 == 2 && w == 2) return launch_geometry<4, 2, 2, true>(a, grid, nq, s, e0, e1);
  if (cb16 == 6 && sb16 == 2 && w == 3) return launch_geometry<6, 2, 3, true>(a, grid, nq, s, e0, e1);
  return TQ_ENOTSUP;
}

int dispatch(const ScoreArgs &a, dim3 grid, int cb16, int sb16, int w, int nq, hipStream_t s, hipEvent_t e0,
             hipEvent_t e1) {
#define TQ_CASE(C, S, W_) \
  if (cb16 == C && sb16 == S && w == W_) return launch_geometry<C, S, W_>(a, grid, nq, s, e0, e1);
  TQ_FOR_EACH_GEOMETRY(TQ_CASE)
#undef TQ_CASE
  return TQ_ENOTSUP;
}

// Records of vectors longer than 256 coordinates: one block per (key group,
// head group) and run of 64-key tiles; the group's A fragments (up to 80 KB at
// d = 1024) are staged in LDS and shared by the block's four waves, and the
// record words are walked in a runtime loop (big_tiles).
struct BigScoreArgs {
  const uint8_t *codes, *signs;
  const float *norms, *rnorms;
  float *logits;
  const uint8_t *ws;
  int64_t T, ldk;
  int qpg, hg, tiles_per_wave, cb16, sb16, nm;
  float alpha;
};

template <int W>
__global__ void __launch_bounds__(256) scores_big_kernel(BigScoreArgs a) {
  extern __shared__ __align__(16) i32x4 Al[];
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, grp = lane >> 4, wv = tid >> 6;
  const int64_t gy = blockIdx.y;                 // key group * hg + head group
  const int64_t kg = gy / a.hg;
  const int hgi = (int)(gy - kg * a.hg);
  const uint8_t *prep = a.ws + gy * prep_stride(a.nm);
  stage_frags(Al, prep, a.nm, tid, 256);
  const HeadConsts hc = HeadConsts::load(reinterpret_cast<const float *>(prep + (int64_t)a.nm * 1024) + grp * 4);
  __syncthreads();
  const int head = hgi * 4 + grp;
  const bool ok = head < a.qpg;
  float *lrow = a.logits + (kg * a.qpg + (ok ? head : 0)) * a.T;
  const int64_t cbytes = 16 * a.cb16, sbytes = 16 * a.sb16;
  const uint8_t *cbase = a.codes + kg * a.ldk * cbytes + grp * a.cb16 * 4;
  const uint8_t *sbase = a.signs + kg * a.ldk * sbytes + grp * a.sb16 * 4;
  const float *nbase = a.norms + kg * a.ldk, *rbase = a.rnorms + kg * a.ldk;
  const int64_t T = a.T;
  const int64_t tile0 = ((int64_t)blockIdx.x * 4 + wv) * a.tiles_per_wave;
  for (int i = 0; i < a.tiles_per_wave; ++i) {
    const int64_t t0 = (tile0 + i) * 64;
    if (t0 >= T) break;
    const uint8_t *cp[4];
    const uint8_t *sp[4];
    float nu[4], ga[4], l[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int64_t t = min(t0 + 16 * s + col, T - 1);
      cp[s] = cbase + t * cbytes;
      sp[s] = sbase + t * sbytes;
      nu[s] = nbase[t];
      ga[s] = rbase[t];
    }
    big_tiles<W, 4>(Al, cp, sp, a.cb16, a.sb16, lane, nu, ga, a.alpha, hc, l);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int64_t t = t0 + 16 * s + col;
      if (ok && t < T) lrow[t] = l[s];
    }
  }
}

int launch_scores_big(const tq_ctx *ctx, const void *ws, int64_t G, int qpg, int64_t T, int64_t ldk,
                      const uint8_t *codes, const uint8_t *signs, const float *norms, const float *rnorms,
                      float *logits, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  BigScoreArgs a{};
  a.codes = codes;
  a.signs = signs;
  a.norms = norms;
  a.rnorms = rnorms;
  a.logits = logits;
  a.ws = reinterpret_cast<const uint8_t *>(ws);
  a.T = T;
  a.ldk = ldk;
  a.qpg = qpg;
  a.hg = (qpg + 3) / 4;
  a.cb16 = ctx->cw16;
  a.sb16 = ctx->sign_bytes / 16;
  a.nm = mfma_count(a.cb16, a.sb16, ctx->hp.w);
  a.alpha = ctx->alpha;
  const int64_t groups = G * a.hg;
  const int64_t tiles = (T + 63) / 64;
  int64_t tpw = (tiles * groups + TQ_SCORES_WAVES - 1) / TQ_SCORES_WAVES;
  if (tpw > (tiles + 3) / 4) tpw = (tiles + 3) / 4;
  if (tpw < 1) tpw = 1;
  const int64_t chunks = (tiles + 4 * tpw - 1) / (4 * tpw);
  if (chunks > 0x7fffffff) return TQ_ENOTSUP;
  a.tiles_per_wave = (int)tpw;
  const size_t lds = (size_t)a.nm * 1024;
  const dim3 grid((unsigned)chunks, (unsigned)groups);
  auto go = [&](auto kern) {
    if (allow_lds(reinterpret_cast<const void *>(kern), lds) != TQ_OK) return TQ_EHIP;
    if (e0 || e1)
      hipExtLaunchKernelGGL(kern, grid, dim3(256), lds, stream, e0, e1, 0, a);
    else
      hipLaunchKernelGGL(kern, grid, dim3(256), lds, stream, a);
    return hip_status();
  };
  return ctx->hp.w == 3 ? go(scores_big_kernel<3>) : go(scores_big_kernel<1>);
}

}  // namespace

int launch_prep(const tq_ctx *ctx, const float *q, int64_t groups, int qpg, int hg, int64_t nq_total,
                uint8_t *ws, hipStream_t stream) {
  if (ctx->hp.d > 256) return launch_prep_big(ctx, q, groups, qpg, hg, nq_total, ws, stream);
  if (prep_gemm_applies(ctx, groups)) return launch_prep_gemm(ctx, q, groups, qpg, hg, nq_total, ws, stream);
  const PrepArgs pa = make_prep_args(ctx, q, qpg, hg, nq_total, ws);
  if (groups > 0x7fffffff) return TQ_ENOTSUP;
  const dim3 grid((unsigned)groups);
  if (pa.d <= 32)
    prep_kernel<32, true><<<grid, PREP_THREADS, 0, stream>>>(pa);
  else if (pa.d <= 64)
    prep_kernel<64, true><<<grid, PREP_THREADS, 0, stream>>>(pa);
  else if (pa.d <= 128)
    prep_kernel<128, true><<<grid, PREP_THREADS, 0, stream>>>(pa);
  else
    prep_kernel<64, false><<<grid, PREP_THREADS, 0, stream>>>(pa);
  return hip_status();
}

size_t scores_ws_bytes(const tq_ctx *ctx, int64_t G, int qpg) {
  const int hg = (qpg + 3) / 4;
  const int nm = mfma_count(ctx->cw16, ctx->sign_bytes / 16, ctx->hp.w);
  return (size_t)(G * hg * prep_stride(nm));
}

int check_scores_shape(const tq_ctx *ctx, int64_t G, int qpg, int64_t T, int64_t ldk) {
  const int64_t groups = G * ((qpg + 3) / 4);
  if (groups > 65535 || T > 0x7fffffff - 64) return TQ_ENOTSUP;
  // per-group record offsets are 32-bit in the scores kernel
  if (ldk * (int64_t)(ctx->code_bytes > ctx->sign_bytes ? ctx->code_bytes : ctx->sign_bytes) >= ((int64_t)1 << 32))
    return TQ_ENOTSUP;
  return TQ_OK;
}

int launch_prep_queries(const tq_ctx *ctx, const float *q, int64_t G, int qpg, void *ws,
                        hipStream_t stream) {
  if (G == 0) return TQ_OK;
  const int hg = (qpg + 3) / 4;
  if (G * hg > 65535) return TQ_ENOTSUP;
  return launch_prep(ctx, q, G * hg, qpg, hg, G * qpg, reinterpret_cast<uint8_t *>(ws), stream);
}

int launch_scores_prepared(const tq_ctx *ctx, const void *ws, int64_t G, int qpg, int64_t T,
                           int64_t ldk, const uint8_t *codes, const uint8_t *signs,
                           const float *norms, const float *rnorms, float *logits,
                           hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (G == 0 || T == 0) return TQ_OK;
  int st = check_scores_shape(ctx, G, qpg, T, ldk);
  if (st != TQ_OK) return st;
  if (ctx->hp.d > 256)
    return launch_scores_big(ctx, ws, G, qpg, T, ldk, codes, signs, norms, rnorms, logits, stream, ev_start,
                             ev_stop);
  const int hg = (qpg + 3) / 4;
  const int cb16 = ctx->cw16, sb16 = ctx->sign_bytes / 16, w = ctx->hp.w;
  // NQ head groups per wave (2 where it fits); blocks along y: key group x NQ-group block
  const int nmc = mfma_count(cb16, sb16, w);
  const int nq = hg >= 4 && nmc <= kScoresNQ4MaxNM && !ctx->frac ? 4 : hg >= 2 && nmc <= kScoresNQ2MaxNM ? 2 : 1;
  const int hq = (hg + nq - 1) / nq;
  const int64_t groups = G * hq;
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
  sa.hq = hq;
  sa.cb = ctx->code_bytes;
  sa.sb = ctx->sign_bytes;
  sa.alpha = ctx->alpha;
  const int spb = kScoresSPB;
  sa.wide = T % spb == 0 && reinterpret_cast<uintptr_t>(logits) % (4 * spb) == 0;
  // key tiles of 16 * spb per wave iteration; aim for ~TQ_SCORES_WAVES waves overall
  const int64_t kt = 16 * spb;
  const int64_t tiles = (T + kt - 1) / kt;
  int64_t tpw = (tiles * groups + TQ_SCORES_WAVES - 1) / TQ_SCORES_WAVES;
  // no more per wave than the four waves of a block share (many head groups
  // over a short context would otherwise leave waves of a block idle)
  if (tpw > (tiles + 3) / 4) tpw = (tiles + 3) / 4;
  if (tpw < 1) tpw = 1;
  if (tpw > 256) tpw = 256;
  const int64_t chunks = (tiles + 4 * tpw - 1) / (4 * tpw);
  sa.tiles_per_wave = (int)tpw;
  if (ctx->frac)
    return dispatch_frac(sa, dim3((unsigned)chunks, (unsigned)groups), cb16, sb16, w, nq, stream, ev_start,
                         ev_stop);
  return dispatch(sa, dim3((unsigned)chunks, (unsigned)groups), cb16, sb16, w, nq, stream, ev_start, ev_stop);
}

int launch_scores(const tq_ctx *ctx, const float *q, int64_t G, int qpg, int64_t T, int64_t ldk,
                  const uint8_t *codes, const uint8_t *signs, const float *norms,
                  const float *rnorms, float *logits, void *ws, hipStream_t stream) {
  if (G == 0 || T == 0) return TQ_OK;
  int st = check_scores_shape(ctx, G, qpg, T, ldk);
  if (st != TQ_OK) return st;
  st = launch_prep_queries(ctx, q, G, qpg, ws, stream);
  if (st != TQ_OK) return st;
  return launch_scores_prepared(ctx, ws, G, qpg, T, ldk, codes, signs, norms, rnorms, logits, stream);
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

// Whole row in registers: one read, one write.  The loads are unconditional
// (clamped index) so that all of them are in flight before the first use; the
// elements past the row end are masked out of the max and the sum.
template <int NT, int VPT>
__global__ void __launch_bounds__(NT) softmax_reg_kernel(const float *in, float *out, int64_t T,
                                                          float scale) {
  const int64_t row = blockIdx.x;
  const float4 *x = reinterpret_cast<const float4 *>(in + row * T);
  float4 *y = reinterpret_cast<float4 *>(out + row * T);
  const int n4 = (int)(T >> 2);
  const int tid = threadIdx.x;
  float4 v[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) v[k] = x[min(tid + k * NT, n4 - 1)];
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    v[k].x *= scale; v[k].y *= scale; v[k].z *= scale; v[k].w *= scale;
    const float mk = fmaxf(fmaxf(v[k].x, v[k].y), fmaxf(v[k].z, v[k].w));
    m = tid + k * NT < n4 ? fmaxf(m, mk) : m;
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    v[k].x = exp2f((v[k].x - m) * kLog2e);
    v[k].y = exp2f((v[k].y - m) * kLog2e);
    v[k].z = exp2f((v[k].z - m) * kLog2e);
    v[k].w = exp2f((v[k].w - m) * kLog2e);
    const float sk = (v[k].x + v[k].y) + (v[k].z + v[k].w);
    s += tid + k * NT < n4 ? sk : 0.f;
  }
  const float mloc = m;
  block_max_sum<NT>(m, s);
  const float f = (mloc == -INFINITY ? 0.f : exp2f((mloc - m) * kLog2e)) / s;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    float4 o = v[k];
    o.x *= f; o.y *= f; o.z *= f; o.w *= f;
    if (tid + k * NT < n4) {
      // streamed out past the caches: their write-back would otherwise
      // compete with the next scores pass
      typedef float f32x4v __attribute__((ext_vector_type(4)));
      __builtin_nontemporal_store(f32x4v{o.x, o.y, o.z, o.w}, reinterpret_cast<f32x4v *>(y) + tid + k * NT);
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
  } else if (vec && T <= TQ_SOFTMAX_NT * 4 * (32768 / 4 / TQ_SOFTMAX_NT)) {
    softmax_reg_kernel<TQ_SOFTMAX_NT, 32768 / 4 / TQ_SOFTMAX_NT><<<g, TQ_SOFTMAX_NT, 0, stream>>>(logits, probs, T, scale);
  } else if (vec && T <= 1024 * 4 * 16) {
    softmax_reg_kernel<1024, 16><<<g, 1024, 0, stream>>>(logits, probs, T, scale);
  } else {
    softmax_stream_kernel<<<g, 1024, 0, stream>>>(logits, probs, T, scale);
  }
  return hip_status();
}

}  // namespace tq
