// Shared pieces of the int8-MFMA estimator (see tq_scores.hip for the math):
// the query-prep interface and the per-16-key tile computation used by the
// scores, top-k and attention kernels.
#pragma once

#include "tq_internal.h"

namespace tq {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Parity words per lane group (3-bit codes): the parity bits of three
// consecutive code words share one word (see ParityMasks).
__host__ __device__ constexpr int parity_words(int cb16, int w) { return w == 3 ? (cb16 + 2) / 3 : 0; }

// MFMAs per 16-key tile: two per 32-bit word (bit planes 0-3, 4-7), over the
// code words, the merged parity words (3-bit codes) and the sign words.
__host__ __device__ inline int mfma_count(int cb16, int sb16, int w) {
  return 2 * cb16 + 2 * parity_words(cb16, w) + 2 * sb16;
}

// bytes of prepared query state per (query group of 4 heads): NM fragments of
// 64 lanes x 16 B, then 4 heads x {1/S_P, 1/S_Q, K_P, K_Q}
__host__ __device__ inline int64_t prep_stride(int nm) {
  return ((int64_t)nm * 1024 + 64 + 255) / 256 * 256;
}

// Build the A fragments for `groups` query groups.  Group i covers queries
// q[(i / hg) * qpg + (i % hg) * 4 + hh], hh < 4, of which those with head
// index < qpg and flat index < nq_total are real (the rest are zero).
int launch_prep(const tq_ctx *ctx, const float *q, int64_t groups, int qpg, int hg,
                int64_t nq_total, uint8_t *ws, hipStream_t stream);

// Record words a lane (column n, lane group g) holds for one key.
template <int CB16, int SB16, int W>
struct KeyWords {
  static constexpr int XW = (W == 3) ? 1 : 0;
  uint32_t cw[CB16 + XW];
  uint32_t sw[SB16];
};

// Streaming keys (scores, attention) are read once per call and are loaded
// with the non-temporal hint: they then do not evict lines that are about to
// be reused, such as the logits a following softmax reads.  A database that
// many query blocks re-read (top-k) uses ordinary loads.
template <bool NT>
__device__ __forceinline__ uint32_t key_word(const uint32_t *p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

// Words of key t for lane group g: uniform base pointers plus 32-bit byte
// offsets (t * record bytes + g * bytes per lane group), so the loads take
// the scalar-base + 32-bit-offset address form with no 64-bit math per lane.
// Words of one key for lane group g, from the lane's first code byte cp and
// first sign byte sp.
template <bool NT, int CB16, int SB16, int W>
__device__ __forceinline__ void load_key_words_at(KeyWords<CB16, SB16, W> &k, const uint8_t *cp,
                                                  const uint8_t *sp, int grp) {
#pragma unroll
  for (int i = 0; i < CB16; ++i) k.cw[i] = key_word<NT>(reinterpret_cast<const uint32_t *>(cp + 4 * i));
  if constexpr (W == 3) {   // first word of the next lane group's chunk (none for the last group)
    const uint32_t nxt = key_word<NT>(reinterpret_cast<const uint32_t *>(cp + 4 * (grp < 3 ? CB16 : CB16 - 1)));
    k.cw[CB16] = grp < 3 ? nxt : 0u;
  }
#pragma unroll
  for (int i = 0; i < SB16; ++i) k.sw[i] = key_word<NT>(reinterpret_cast<const uint32_t *>(sp + 4 * i));
}

template <bool NT, int CB16, int SB16, int W>
__device__ __forceinline__ void load_key_words(KeyWords<CB16, SB16, W> &k, const uint8_t *cbase,
                                               const uint8_t *sbase, uint32_t t, int grp) {
  const uint32_t co = t * (CB16 * 16) + (uint32_t)grp * (CB16 * 4);
  const uint32_t so = t * (SB16 * 16) + (uint32_t)grp * (SB16 * 4);
  load_key_words_at<NT>(k, cbase + co, sbase + so, grp);
}

// base[i] with a 32-bit byte offset (scalar base + 32-bit offset address form)
__device__ __forceinline__ float load_f32(const float *base, uint32_t i) {
  return *reinterpret_cast<const float *>(reinterpret_cast<const uint8_t *>(base) + i * 4u);
}

__device__ __forceinline__ i32x4 mfma8(const i32x4 &a, const i32x4 &b, const i32x4 &c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// bit planes 4*half .. 4*half+3 of each byte of w, as int8 values 2^j (-128 for j = 7)
__device__ __forceinline__ i32x4 planes(uint32_t w, int half) {
  const int s = 4 * half;
  return i32x4{(int)(w & (0x01010101u << s)), (int)(w & (0x01010101u << (s + 1))),
               (int)(w & (0x01010101u << (s + 2))), (int)(w & (0x01010101u << (s + 3)))};
}

// Per-head constants of the prepared query: 1/S_P and 1/S_Q (scaled by 2^-7
// for the digit-pair recombination of tile_logit), K_P and K_Q.
struct HeadConsts {
  float invSP, invSQ, KP, KQ;
  __device__ static HeadConsts load(const float *cst) {
    return HeadConsts{cst[0] * 0x1.0p-7f, cst[1] * 0x1.0p-7f, cst[2], cst[3]};
  }
};

template <int CB16, int SB16, int W>
struct ScoreShape {
  static constexpr int NPW = parity_words(CB16, W);
  static constexpr int NMC = 2 * CB16, NMP = 2 * NPW, NMS = 2 * SB16;
  static constexpr int NM = NMC + NMP + NMS;
};

// 3-bit codes are packed back to back, so code k starts at record bit 3k.
// Lane group g holds record words g*CB16 .. g*CB16+CB16-1; since 32 = 2 (mod 3),
// a code starts at bit q of record word r exactly when q = r (mod 3).  The
// parity words of three consecutive record words therefore carry their
// code-start bits on three disjoint residues, and are merged into one word
// with the masks m[p] (bits q = g*CB16+p mod 3); bits elsewhere (parities of
// windows that are not codes) are dropped.  The A fragments of a merged word
// carry, for bit q, the weight of the code that starts there.
template <int CB16, int W>
struct ParityMasks {
  uint32_t m[W == 3 ? CB16 : 1];
};
template <int CB16, int W>
__device__ __forceinline__ ParityMasks<CB16, W> parity_masks(int grp) {
  ParityMasks<CB16, W> pm{};
  if constexpr (W == 3) {
#pragma unroll
    for (int p = 0; p < CB16; ++p) pm.m[p] = 0x49249249u << ((grp * CB16 + p) % 3);
  }
  return pm;
}

// Logits of head (lane / 16) of NQ query groups (A[g], hc[g]) for key
// (lane % 16) of the tile:  nu * (P + alpha * gamma * Q), P and Q recombined
// from four int32 digit rows.  Each bit-plane operand is built once and used
// by the NQ groups' MFMAs.
//
// FRAC: fractional-width records (planar quarters): lane group g holds the
// bit planes of its quarter's codes, CB16 = 3 WPP words for 3-bit codes, and
// a code's parity is the XOR of its three plane words (no merging).
template <int CB16, int SB16, int W, int NQ, bool FRAC = false>
__device__ __forceinline__ void tile_logits(const i32x4 (*A)[ScoreShape<CB16, SB16, W>::NM],
                                            const KeyWords<CB16, SB16, W> &k, float nu, float gamma,
                                            float alpha, const HeadConsts *hc,
                                            const ParityMasks<CB16, W> &pm, float *out) {
  using Sh = ScoreShape<CB16, SB16, W>;
  i32x4 accP[NQ], accQ[NQ];
#pragma unroll
  for (int g = 0; g < NQ; ++g) accP[g] = accQ[g] = i32x4{0, 0, 0, 0};
  auto mf = [&](i32x4 (&acc)[NQ], int mu, uint32_t word, int half) {
    const i32x4 b = planes(word, half);
#pragma unroll
    for (int g = 0; g < NQ; ++g) acc[g] = mfma8(A[g][mu], b, acc[g]);
  };
#pragma unroll
  for (int p = 0; p < CB16; ++p) {
    mf(accP, 2 * p, k.cw[p], 0);
    mf(accP, 2 * p + 1, k.cw[p], 1);
  }
  if constexpr (W == 3 && FRAC) {
    constexpr int WPP = CB16 / 3;
    static_assert(Sh::NPW == WPP, "one parity word per plane word");
#pragma unroll
    for (int f = 0; f < WPP; ++f) {
      const uint32_t pw = k.cw[f] ^ k.cw[WPP + f] ^ k.cw[2 * WPP + f];
      mf(accP, Sh::NMC + 2 * f, pw, 0);
      mf(accP, Sh::NMC + 2 * f + 1, pw, 1);
    }
  } else if constexpr (W == 3) {
    // bit q of par = parity of record bits q, q+1, q+2
    uint32_t pw[Sh::NPW];
#pragma unroll
    for (int p = 0; p < CB16; ++p) {
      const uint32_t lo = k.cw[p], hi = k.cw[p + 1];
      const uint32_t par = lo ^ __builtin_amdgcn_alignbit(hi, lo, 1) ^ __builtin_amdgcn_alignbit(hi, lo, 2);
      pw[p / 3] = (p % 3 == 0) ? (par & pm.m[p]) : (pw[p / 3] | (par & pm.m[p]));
    }
#pragma unroll
    for (int f = 0; f < Sh::NPW; ++f) {
      mf(accP, Sh::NMC + 2 * f, pw[f], 0);
      mf(accP, Sh::NMC + 2 * f + 1, pw[f], 1);
    }
  }
#pragma unroll
  for (int p = 0; p < SB16; ++p) {
    mf(accQ, Sh::NMC + Sh::NMP + 2 * p, k.sw[p], 0);
    mf(accQ, Sh::NMC + Sh::NMP + 2 * p + 1, k.sw[p], 1);
  }
  // digits recombined in pairs in int32 (d0*128 + d1 and d2*128 + d3; every
  // |digit sum| < 2^22 for records of up to 256 coordinates, so the pairs
  // stay below 2^30), then in fp32; invSP and invSQ carry the 2^-7 of the
  // leading pair (HeadConsts::load)
  const float ag = alpha * gamma;
#pragma unroll
  for (int g = 0; g < NQ; ++g) {
    const float P = fmaf(fmaf((float)(accP[g][2] * 128 + accP[g][3]), 0x1.0p-14f,
                              (float)(accP[g][0] * 128 + accP[g][1])),
                         hc[g].invSP, -hc[g].KP);
    const float Q = fmaf(fmaf((float)(accQ[g][2] * 128 + accQ[g][3]), 0x1.0p-14f,
                              (float)(accQ[g][0] * 128 + accQ[g][1])),
                         hc[g].invSQ, -hc[g].KQ);
    out[g] = nu * fmaf(ag, Q, P);
  }
}

// One query group's logit (tile_logits with NQ = 1).
template <int CB16, int SB16, int W>
__device__ __forceinline__ float tile_logit(const i32x4 *A, const KeyWords<CB16, SB16, W> &k, float nu,
                                            float gamma, float alpha, const HeadConsts &hc,
                                            const ParityMasks<CB16, W> &pm) {
  float l;
  tile_logits<CB16, SB16, W, 1>(reinterpret_cast<const i32x4 (*)[ScoreShape<CB16, SB16, W>::NM]>(A), k, nu,
                                gamma, alpha, &hc, pm, &l);
  return l;
}

// s_waitcnt vmcnt(N): at most N vector memory instructions of this wave still
// outstanding (loads complete in issue order, so every load issued more than
// N loads ago has landed).  The copies into LDS (global_load_lds) are waited
// for this way, explicitly: the compiler does not order them before later
// LDS reads of the same slot.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}

// Wave-wide sum / max with DPP row permutes (quad swaps, half-row and row
// mirrors make every lane of a 16-lane row hold the row result) and four
// readlanes; much shorter latency than a chain of ds_bpermute shuffles.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_sum(float v) {
  v += dpp_f<0xb1>(v);    // quad_perm [1,0,3,2]
  v += dpp_f<0x4e>(v);    // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);   // row_half_mirror
  v += dpp_f<0x140>(v);   // row_mirror
  return v;
}
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, dpp_f<0xb1>(v));
  v = fmaxf(v, dpp_f<0x4e>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return v;
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = row_max(v);
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

// Records of any geometry (vectors longer than 256 coordinates, or callers
// that keep no per-geometry kernel): the record words are read one at a
// time in a runtime loop and the A fragments come from LDS (Al = [nm][64]),
// where the 4 waves of a block share them.  NK 16-key tiles are scored per
// pass, so that every fragment read from LDS serves NK MFMAs.  cp[s] / sp[s]
// point at the lane's first code / sign word of its key in tile s (lane
// group g: record words g*cb16 .. g*cb16 + cb16 - 1).  The digit rows are
// recombined in fp32 (their int32 sums reach ~2^24 at d = 1024, so the
// int32 pair recombination of tile_logits could overflow).
template <int W, int NK>
__device__ __forceinline__ void big_tiles(const i32x4 *Al, const uint8_t *const (&cp)[NK],
                                          const uint8_t *const (&sp)[NK], int cb16, int sb16, int lane,
                                          const float (&nu)[NK], const float (&ga)[NK], float alpha,
                                          const HeadConsts &hc, float (&out)[NK]) {
  const int grp = lane >> 4;
  i32x4 accP[NK], accQ[NK];
#pragma unroll
  for (int s = 0; s < NK; ++s) accP[s] = accQ[s] = i32x4{0, 0, 0, 0};
  const int nmc = 2 * cb16, nmp = 2 * parity_words(cb16, W);
  uint32_t cur[NK], pw[NK];
#pragma unroll
  for (int s = 0; s < NK; ++s) {
    cur[s] = *reinterpret_cast<const uint32_t *>(cp[s]);
    pw[s] = 0u;
  }
  for (int p = 0; p < cb16; ++p) {
    // the word after this one: the next lane group's first word after the
    // last (3-bit codes cross words), none for the last lane group
    const bool has_next = p + 1 < cb16 || (W == 3 && grp < 3);
    uint32_t nxt[NK];
#pragma unroll
    for (int s = 0; s < NK; ++s) nxt[s] = has_next ? *reinterpret_cast<const uint32_t *>(cp[s] + 4 * (p + 1)) : 0u;
    const i32x4 a0 = Al[(2 * p) * 64 + lane], a1 = Al[(2 * p + 1) * 64 + lane];
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      accP[s] = mfma8(a0, planes(cur[s], 0), accP[s]);
      accP[s] = mfma8(a1, planes(cur[s], 1), accP[s]);
    }
    if constexpr (W == 3) {
      const uint32_t mask = 0x49249249u << ((grp * cb16 + p) % 3);
#pragma unroll
      for (int s = 0; s < NK; ++s) {
        const uint32_t par = cur[s] ^ __builtin_amdgcn_alignbit(nxt[s], cur[s], 1) ^
                             __builtin_amdgcn_alignbit(nxt[s], cur[s], 2);
        pw[s] |= par & mask;
      }
      if (p % 3 == 2 || p == cb16 - 1) {
        const int f = p / 3;
        const i32x4 a2 = Al[(nmc + 2 * f) * 64 + lane], a3 = Al[(nmc + 2 * f + 1) * 64 + lane];
#pragma unroll
        for (int s = 0; s < NK; ++s) {
          accP[s] = mfma8(a2, planes(pw[s], 0), accP[s]);
          accP[s] = mfma8(a3, planes(pw[s], 1), accP[s]);
          pw[s] = 0u;
        }
      }
    }
#pragma unroll
    for (int s = 0; s < NK; ++s) cur[s] = nxt[s];
  }
  for (int p = 0; p < sb16; ++p) {
    const i32x4 a0 = Al[(nmc + nmp + 2 * p) * 64 + lane], a1 = Al[(nmc + nmp + 2 * p + 1) * 64 + lane];
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      const uint32_t wd = *reinterpret_cast<const uint32_t *>(sp[s] + 4 * p);
      accQ[s] = mfma8(a0, planes(wd, 0), accQ[s]);
      accQ[s] = mfma8(a1, planes(wd, 1), accQ[s]);
    }
  }
#pragma unroll
  for (int s = 0; s < NK; ++s) {
    const float Ph = fmaf((float)accP[s][0], 128.f, (float)accP[s][1]);
    const float Pl = fmaf((float)accP[s][2], 128.f, (float)accP[s][3]);
    const float Qh = fmaf((float)accQ[s][0], 128.f, (float)accQ[s][1]);
    const float Ql = fmaf((float)accQ[s][2], 128.f, (float)accQ[s][3]);
    const float P = fmaf(fmaf(Pl, 0x1.0p-14f, Ph), hc.invSP, -hc.KP);
    const float Q = fmaf(fmaf(Ql, 0x1.0p-14f, Qh), hc.invSQ, -hc.KQ);
    out[s] = nu[s] * fmaf(alpha * ga[s], Q, P);
  }
}

// Copies one query group's A fragments (nm x 64 lanes x 16 B, at prep) into
// LDS with all threads of a block of nthreads.
__device__ __forceinline__ void stage_frags(i32x4 *Al, const uint8_t *prep, int nm, int tid, int nthreads) {
  const i32x4 *src = reinterpret_cast<const i32x4 *>(prep);
  for (int i = tid; i < nm * 64; i += nthreads) Al[i] = src[i];
}

// Expands a dispatch over the record geometries d <= 256 can produce:
// (code words per lane group, sign words per lane group, code bits).
#define TQ_FOR_EACH_GEOMETRY(X)                                              \
  X(1, 1, 1) X(2, 2, 1)                                           \
  X(1, 1, 2) X(2, 1, 2) X(3, 2, 2) X(4, 2, 2)                                \
  X(1, 1, 3) X(2, 1, 3) X(3, 1, 3) X(4, 2, 3) X(5, 2, 3) X(6, 2, 3)

}  // namespace tq
