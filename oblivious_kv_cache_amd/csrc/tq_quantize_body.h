// Quantize kernel body: norm, rotation, scalar codes, residual, QJL sign sketch.
//
// Per vector x (xujun.org note 189244, sections 第一步：PolarQuant and
// 第二步：QJL; suzuke blog "turboquant-compressing-ai-consciousness",
// 技術上怎麼做到的, 第一步 to 第三步):
//   nu = |x|,  y = Pi x / nu,  idx_i = #{k : t_k < y_i},  r = y - c[idx],
//   gamma = |r|,  bit_j = [(S' r)_j >= 0] with S' = S Pi^T.
//
// Mapping onto CDNA4: both products are GEMMs over a tile of vectors and run
// on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  The operands that are
// not exactly representable in bf16 are split into hi + lo bf16 parts, which
// keeps every product to about 2^-17 relative error so that a code or sign
// flips only for coordinates within ~1e-5 of a decision boundary:
//   GEMM 1 (Y^T = Pi X^T): Pi_hi x + Pi_lo x  (bf16 x is exact), plus
//                          Pi_hi x_lo for fp32 inputs;
//   GEMM 2 (Z^T = S' R^T): S'_hi r_hi + S'_hi r_lo + S'_lo r_hi.
// A lane of the 16x16 accumulator holds 4 rows of one column.  The rows of Pi
// and S' are permuted on the host so that lane group g (= lane / 16) ends up
// with the contiguous coordinate range [g d/4, (g+1) d/4) of its vector: the
// codebook search, the bit packing and the GEMM-2 operand (the residual) all
// stay in that lane's registers, and each lane stores one contiguous run of
// code bytes and sign bytes.
#pragma once

#include "tq_internal.h"

namespace tq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Bits collected by shifting each value's sign bit in at the bottom (one
// alignbit per value, first value ends highest) -> bit i = NOT sign of value
// i, i < n: reversed, moved down and inverted.
template <int N>
__device__ __forceinline__ uint32_t nonneg_bits(uint32_t shifted) {
  const uint32_t r = __builtin_bitreverse32(shifted) >> (32 - N);
  return r ^ (N == 32 ? 0xffffffffu : ((1u << N) - 1u));
}
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct QArgs {
  const void *x;
  int64_t n, ldx, ldr, ntiles;
  uint8_t *codes, *signs;
  float *norms, *rnorms;
  const Frag *PiA_hi, *PiA_lo, *S2A_hi, *S2A_lo;
  int d, m, prod, code_bytes, sign_bytes;
  float tpos[8], cpos[8];
};

__device__ __forceinline__ bf16x8 as_bf(const Frag &f) { return __builtin_bit_cast(bf16x8, f); }

__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Store nb bytes held little-endian in words[] at dst (any alignment).
template <int NW>
__device__ __forceinline__ void store_bytes(uint8_t *dst, const uint32_t (&words)[NW], int nb) {
  if (nb <= 0) return;
  if ((((uintptr_t)dst) & 3) == 0 && (nb & 3) == 0) {
    uint32_t *d32 = reinterpret_cast<uint32_t *>(dst);
#pragma unroll
    for (int i = 0; i < NW; ++i)
      if (4 * i < nb) d32[i] = words[i];
  } else {
#pragma unroll
    for (int i = 0; i < 4 * NW; ++i)
      if (i < nb) dst[i] = (uint8_t)(words[i >> 2] >> (8 * (i & 3)));
  }
}

__device__ __forceinline__ void zero_bytes(uint8_t *dst, int nb) {
  for (int i = 0; i < nb; ++i) dst[i] = 0;
}

// The kernel body, callable from a kernel that also runs other jobs: block
// `block` of `nblocks` blocks of NTHR threads working on this quantize job;
// `lds` holds the operand fragments (USE_LDS: 4 FR x 64 Frags, filled here by
// the block's NTHR threads).
//
// PLANES (MSE-only contexts): the codes are stored as W bit planes of d bits
// (plane p in record bytes [p d/8, (p+1) d/8), bit p of code i at bit i), so
// a lane holds PW words per plane for its PER coordinates and stores PER/8
// bytes into each plane.  (With W = 1 both layouts are the same.)
template <int DPAD, bool BF16IN, bool USE_LDS, int NTL, int W, bool FULL, int NTHR, bool PLANES = false>
__device__ __forceinline__ void quantize_body(const QArgs &a, Frag *lds, int block, int nblocks) {
  constexpr int NT = DPAD / 16;       // 16-row output tiles (coordinates)
  constexpr int NK = DPAD / 32;       // 32-deep k blocks
  constexpr int FR = NT * NK;         // operand fragments per matrix
  constexpr int PER = DPAD / 4;       // coordinates (and sketch rows) per lane
  constexpr int HALF = (1 << W) / 2;  // L / 2
  constexpr bool PL = PLANES && W > 1;
  constexpr int PW = (PER + 31) / 32;       // words per bit plane (PL)
  constexpr int CW = PL ? W * PW : (PER * W + 31) / 32;   // code words per lane
  constexpr int SW = (PER + 31) / 32;       // sign words per lane
  constexpr int CBYTES = PER * W / 8;       // code bytes per lane (whole bytes: PER % 8 == 0)
  constexpr int SBYTES = PER / 8;
  // d == DPAD (and m == d): when the lane groups' byte runs are whole dwords
  // and together fill a 16-byte-multiple record, the record has no padding
  // and every lane stores plain dwords
  constexpr bool CEXACT = FULL && CBYTES % 4 == 0 && (4 * CBYTES) % 16 == 0;
  constexpr bool SEXACT = FULL && SBYTES % 4 == 0 && (4 * SBYTES) % 16 == 0;

  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;

  if constexpr (USE_LDS) {
    // Fill LDS with one batch of independent 16-byte loads per thread over
    // all operand matrices (each matrix pointer stays a scalar; choosing it
    // with a runtime index would re-load it from the kernel arguments), then
    // store: one memory round trip.  Clamped indices keep the loads free of
    // branches; a duplicate store of the last element rewrites the same value.
    constexpr int NF = FR * 64;
    constexpr int ITER = (NF + NTHR - 1) / NTHR;
    // Without the sketch (MSE-only contexts) slots 2 and 3 receive a second
    // copy of Pi's fragments, unused: the loads stay unconditional.
    const Frag *const s0 = a.PiA_hi, *const s1 = a.PiA_lo;
    const Frag *const s2 = a.prod ? a.S2A_hi : a.PiA_hi, *const s3 = a.prod ? a.S2A_lo : a.PiA_lo;
    Frag t0[ITER], t1[ITER], t2[ITER], t3[ITER];
#pragma unroll
    for (int b = 0; b < ITER; ++b) {
      const int i = min(b * NTHR + (int)threadIdx.x, NF - 1);
      t0[b] = s0[i];
      t1[b] = s1[i];
      t2[b] = s2[i];
      t3[b] = s3[i];
    }
#pragma unroll
    for (int b = 0; b < ITER; ++b) {
      const int i = min(b * NTHR + (int)threadIdx.x, NF - 1);
      lds[i] = t0[b];
      lds[NF + i] = t1[b];
      lds[2 * NF + i] = t2[b];
      lds[3 * NF + i] = t3[b];
    }
    __syncthreads();
  }
  // Fragment f of operand matrix `which` for this lane.  `lofs` is re-made
  // opaque in every tile iteration so that address arithmetic for all
  // fragments is not hoisted out of the loop into registers.
  int lofs = lane;
  // second base for matrices 2 and 3 (the S' fragments): every fragment then
  // lies within the 64 KB immediate-offset reach of one of the two bases
  int lofs2 = lane + 2 * FR * 64;
  const Frag *const PiH = a.PiA_hi, *const PiL = a.PiA_lo, *const S2H = a.S2A_hi, *const S2L = a.S2A_lo;
  auto frag = [&](int which, int f) -> bf16x8 {
    if constexpr (USE_LDS) {
      return as_bf(which < 2 ? lds[(which * FR + f) * 64 + lofs] : lds[((which - 2) * FR + f) * 64 + lofs2]);
    } else {
      const Frag *src = which == 0 ? PiH : which == 1 ? PiL : which == 2 ? S2H : S2L;
      return as_bf(src[f * 64 + lofs]);
    }
  };

  const int64_t wave = ((int64_t)block * NTHR + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)nblocks * NTHR) >> 6;

  for (int64_t tile = wave; tile < a.ntiles; tile += nwaves) {
    // The operand fragments are loop-invariant; a memory clobber per tile keeps
    // the compiler from hoisting all of them into registers.
    __asm__ volatile("" ::: "memory");
    // Number of real coordinates / sketch rows in this lane's range.  Kept
    // opaque so the per-coordinate compares are not hoisted out of the loop.
    int nval = a.d - grp * PER, mval = a.m - grp * PER, xval = a.d - grp * 8;
    lofs = lane;
    lofs2 = lane + 2 * FR * 64;
    __asm__ volatile("" : "+v"(nval), "+v"(mval), "+v"(xval), "+v"(lofs), "+v"(lofs2));
    const int64_t vbase = tile * (16 * NTL);
    bf16x8 bx[NTL][NK];
    bf16x8 bxl[NTL][BF16IN ? 1 : NK];
    double ss[NTL];
    int64_t vi[NTL];
    bool valid[NTL];
#pragma unroll
    for (int t = 0; t < NTL; ++t) {
      vi[t] = vbase + t * 16 + col;
      valid[t] = vi[t] < a.n;
      ss[t] = 0.0;
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        const int j0 = k * 32 + grp * 8;
        const bool in = valid[t] && (FULL || k * 32 < xval);   // j0 < d
        if constexpr (BF16IN) {
          Frag f = {{0u, 0u, 0u, 0u}};
          if (in) f = *reinterpret_cast<const Frag *>(
                      reinterpret_cast<const uint16_t *>(a.x) + vi[t] * a.ldx + j0);
          bx[t][k] = as_bf(f);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const double v = (double)(float)bx[t][k][e];
            ss[t] += v * v;
          }
        } else {
          float4 lo4 = make_float4(0.f, 0.f, 0.f, 0.f), hi4 = lo4;
          if (in) {
            const float4 *p = reinterpret_cast<const float4 *>(
                reinterpret_cast<const float *>(a.x) + vi[t] * a.ldx + j0);
            lo4 = p[0];
            hi4 = p[1];
          }
          const float xs[8] = {lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const __bf16 h = (__bf16)xs[e];
            bx[t][k][e] = h;
            bxl[t][k][e] = (__bf16)(xs[e] - (float)h);
            ss[t] += (double)xs[e] * (double)xs[e];
          }
        }
      }
      ss[t] += __shfl_xor(ss[t], 16);
      ss[t] += __shfl_xor(ss[t], 32);
    }
    // A vector shorter than 2^-64 is rotated as x * 2^64 (exact: a power of
    // two), so that neither its inputs nor the products of the rotation fall
    // into the float32 denormal range and 1/nu cannot overflow; nu itself is
    // the unscaled length.  Such vectors are rare, so the wave takes this
    // branch only when one of its lanes has one.
    float xsc[NTL];
    bool any_tiny = false;
#pragma unroll
    for (int t = 0; t < NTL; ++t) {
      const bool tiny = ss[t] > 0.0 && ss[t] < 0x1.0p-128;
      xsc[t] = tiny ? 0x1.0p64f : 1.f;
      any_tiny |= tiny;
    }
    if (__builtin_amdgcn_ballot_w64(any_tiny) != 0) {
#pragma unroll
      for (int t = 0; t < NTL; ++t) {
#pragma unroll
        for (int k = 0; k < NK; ++k) {
          if constexpr (BF16IN) {
#pragma unroll
            for (int e = 0; e < 8; ++e) bx[t][k][e] = (__bf16)((float)bx[t][k][e] * xsc[t]);
          } else {
            // the hi/lo split is redone from the scaled float32 inputs
            const int j0 = k * 32 + grp * 8;
            const bool in = valid[t] && (FULL || k * 32 < xval);
            float4 lo4 = make_float4(0.f, 0.f, 0.f, 0.f), hi4 = lo4;
            if (in) {
              const float4 *p = reinterpret_cast<const float4 *>(
                  reinterpret_cast<const float *>(a.x) + vi[t] * a.ldx + j0);
              lo4 = p[0];
              hi4 = p[1];
            }
            const float xs[8] = {lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float v = xs[e] * xsc[t];
              const __bf16 h = (__bf16)v;
              bx[t][k][e] = h;
              bxl[t][k][e] = (__bf16)(v - (float)h);
            }
          }
        }
      }
    }

    // Per vector: 1/nu, and state for the codes and the residual.
    uint32_t cw[NTL][CW];
    u32x4 rh[NTL][NK], rl[NTL][NK];      // residual hi / lo, bf16 pairs
    float nu[NTL], inv[NTL], rs[NTL];
#pragma unroll
    for (int t = 0; t < NTL; ++t) {
      const double nud = sqrt(ss[t]);
      nu[t] = (float)nud;
      inv[t] = nud > 0.0 ? (float)(1.0 / (nud * (double)xsc[t])) : 0.f;
      rs[t] = 0.f;
#pragma unroll
      for (int i = 0; i < CW; ++i) cw[t][i] = 0u;
    }

    // GEMM 1, one 16-coordinate output tile at a time, each tile consumed by
    // the codebook search while the MFMAs of the next tile run: the search's
    // VALU instructions are interleaved with those MFMAs (one MFMA, then a
    // few VALU instructions), so the matrix cores and the VALU work at once
    // within the wave.
    auto gemm1 = [&](int u, f32x4 (&acc)[NTL]) {
#pragma unroll
      for (int t = 0; t < NTL; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        const bf16x8 ah = frag(0, u * NK + k), al = frag(1, u * NK + k);
#pragma unroll
        for (int t = 0; t < NTL; ++t) {
          acc[t] = mfma(ah, bx[t][k], acc[t]);
          acc[t] = mfma(al, bx[t][k], acc[t]);
          if constexpr (!BF16IN) acc[t] = mfma(ah, bxl[t][k], acc[t]);
        }
      }
    };
    constexpr int G1_MFMA = NK * NTL * (BF16IN ? 2 : 3);   // MFMAs per output tile
    f32x4 accs[2][NTL];
    gemm1(0, accs[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      f32x4 (&acc)[NTL] = accs[u & 1];
      if (u + 1 < NT) gemm1(u + 1, accs[(u + 1) & 1]);
#pragma unroll
      for (int t = 0; t < NTL; ++t) {
        float rr[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int li = 4 * u + jj;                 // local coordinate index
          const float y = acc[t][jj] * inv[t];
          const uint32_t yb = __float_as_uint(y), ab = yb & 0x7fffffffu;
          // codebook search on |y| against the positive thresholds
          uint32_t mm = 0;
          float cm = a.cpos[0];
#pragma unroll
          for (int j = 0; j < HALF - 1; ++j) {
            const bool gt = __uint_as_float(ab) > a.tpos[j];
            mm += gt ? 1u : 0u;
            cm = gt ? a.cpos[j + 1] : cm;
          }
          const uint32_t cmb = __float_as_uint(cm);
          // r = y - copysign(c, y); the sign of y picks the half of the
          // codebook: idx = HALF + mm for y >= +0, its mirror HALF - 1 - mm
          // (= (HALF + mm) ^ (2 HALF - 1)) for y <= -0.  (y == +0 exactly lies
          // on the middle threshold, inside the decision band.)
          float r = y - __uint_as_float(cmb | (yb & 0x80000000u));
          if constexpr (W == 1) {
            // idx = NOT sign bit: collected with one alignbit, fixed per word below
            cw[t][li >> 5] = __builtin_amdgcn_alignbit(cw[t][li >> 5], yb, 31);
          } else {
            const uint32_t neg = (uint32_t)((int32_t)yb >> 31);     // all ones for y <= -0
            uint32_t idx = ((uint32_t)HALF + mm) ^ (neg & (uint32_t)(2 * HALF - 1));
            if constexpr (!FULL) {
              if (li >= nval) idx = 0u;      // padding coordinates
            }
            if constexpr (PL) {
#pragma unroll
              for (int pl = 0; pl < W; ++pl) {
                cw[t][pl * PW + (li >> 5)] |= ((idx >> pl) & 1u) << (li & 31);
                __asm__ volatile("" : "+v"(cw[t][pl * PW + (li >> 5)]));
              }
            } else {
              const int bit = li * W;
              cw[t][bit >> 5] |= idx << (bit & 31);
              if (((bit & 31) + W) > 32) cw[t][(bit >> 5) + 1] |= idx >> (32 - (bit & 31));
              // packed here and now (an empty asm reads the word): otherwise the
              // search results of many coordinates stay live, as lane masks in
              // scalar registers, until the compiler's chosen packing spot, and
              // spill
              __asm__ volatile("" : "+v"(cw[t][bit >> 5]));
            }
          }
          if constexpr (!FULL) {
            if (li >= nval) r = 0.f;
          }
          rs[t] += r * r;
          rr[jj] = r;
        }
        // hi / lo bf16 split of the residual, two coordinates per conversion
#pragma unroll
        for (int jj = 0; jj < 4; jj += 2) {
          const int li = 4 * u + jj;
          const uint32_t hw = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{rr[jj], rr[jj + 1]}, bf16x2));
          const float h0 = __uint_as_float(hw << 16), h1 = __uint_as_float(hw & 0xffff0000u);
          const uint32_t lw = __builtin_bit_cast(uint32_t,
                                                 __builtin_convertvector(f32x2{rr[jj] - h0, rr[jj + 1] - h1}, bf16x2));
          rh[t][li >> 3][(li & 7) >> 1] = hw;
          rl[t][li >> 3][(li & 7) >> 1] = lw;
        }
      }
      if (u + 1 < NT) {
        // the next tile's fragment reads first, then MFMA / VALU alternating
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * NK, 0);    // DS reads
#pragma unroll
        for (int i = 0; i < G1_MFMA; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);       // VALU
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // keep fragment loads from piling up
    }

    if constexpr (W == 1) {
#pragma unroll
      for (int t = 0; t < NTL; ++t)
#pragma unroll
        for (int i = 0; i < CW; ++i) {
          constexpr int NB = PER < 32 ? PER : 32;   // PER is 32 or less, or a multiple of 32
          uint32_t v = nonneg_bits<NB>(cw[t][i]);
          if constexpr (!FULL) {                    // padding coordinates get code 0
            const int nv = nval - 32 * i;
            v &= nv >= 32 ? 0xffffffffu : (nv > 0 ? (1u << nv) - 1u : 0u);
          }
          cw[t][i] = v;
        }
    }
    // a zero vector stores zero codes and gamma = 0 (its signs are cleared below)
#pragma unroll
    for (int t = 0; t < NTL; ++t) {
      if (!(nu[t] > 0.f)) {
#pragma unroll
        for (int i = 0; i < CW; ++i) cw[t][i] = 0u;
        rs[t] = 0.f;
      }
    }
#pragma unroll
    for (int t = 0; t < NTL; ++t) {
      rs[t] += __shfl_xor(rs[t], 16);
      rs[t] += __shfl_xor(rs[t], 32);
      if (valid[t]) {
        uint8_t *rec = a.codes + vi[t] * a.ldr * a.code_bytes;
        const int off = grp * CBYTES;
        if constexpr (PL) {
          // plane pl: this lane group's PER bits at record bit pl d + grp PER
          // (the bytes of real coordinates only; d is a multiple of 8)
          const int pb = a.d >> 3, nb = min(PER / 8, max(0, pb - grp * (PER / 8)));
#pragma unroll
          for (int pl = 0; pl < W; ++pl)
            store_bytes<PW>(rec + pl * pb + grp * (PER / 8),
                            *reinterpret_cast<const uint32_t(*)[PW]>(&cw[t][pl * PW]), nb);
          if (grp == 3 && W * pb < a.code_bytes) zero_bytes(rec + W * pb, a.code_bytes - W * pb);
        } else if constexpr (CEXACT) {
          // the 4 lane groups' byte runs tile the record exactly, dword-aligned
#pragma unroll
          for (int i = 0; i < CBYTES / 4; ++i) reinterpret_cast<uint32_t *>(rec + off)[i] = cw[t][i];
        } else {
          store_bytes<CW>(rec + off, cw[t], min(CBYTES, a.code_bytes - off));
          if (grp == 3 && 4 * CBYTES < a.code_bytes) zero_bytes(rec + 4 * CBYTES, a.code_bytes - 4 * CBYTES);
        }
        if (grp == 0) a.norms[vi[t] * a.ldr] = nu[t];
      }
    }

    if (a.prod) {
      // GEMM 2 (JL sketch of the residual), one 16-row output tile at a time.
      uint32_t sw[NTL][SW];
#pragma unroll
      for (int t = 0; t < NTL; ++t)
#pragma unroll
        for (int i = 0; i < SW; ++i) sw[t][i] = 0u;
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        f32x4 z[NTL];
#pragma unroll
        for (int t = 0; t < NTL; ++t) z[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < NK; ++k) {
          const bf16x8 sh = frag(2, u * NK + k), sl = frag(3, u * NK + k);
#pragma unroll
          for (int t = 0; t < NTL; ++t) {
            const bf16x8 bh = __builtin_bit_cast(bf16x8, rh[t][k]), bl = __builtin_bit_cast(bf16x8, rl[t][k]);
            z[t] = mfma(sh, bh, z[t]);
            z[t] = mfma(sh, bl, z[t]);
            z[t] = mfma(sl, bh, z[t]);
          }
        }
#pragma unroll
        for (int t = 0; t < NTL; ++t) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            // bit = [z >= 0] = NOT sign of z (z is never -0: the sums start at
            // +0); collected with one alignbit, fixed per word below
            const int li = 4 * u + jj;
            sw[t][li >> 5] = __builtin_amdgcn_alignbit(sw[t][li >> 5], __float_as_uint(z[t][jj]), 31);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int t = 0; t < NTL; ++t) {
#pragma unroll
        for (int i = 0; i < SW; ++i) {
          constexpr int NB = PER < 32 ? PER : 32;
          uint32_t v = nonneg_bits<NB>(sw[t][i]);
          if constexpr (!FULL) {                    // rows past m are 0
            const int mv = mval - 32 * i;
            v &= mv >= 32 ? 0xffffffffu : (mv > 0 ? (1u << mv) - 1u : 0u);
          }
          sw[t][i] = v;
        }
        if (!(nu[t] > 0.f)) {
#pragma unroll
          for (int i = 0; i < SW; ++i) sw[t][i] = 0u;
        }
        if (valid[t]) {
          uint8_t *rec = a.signs + vi[t] * a.ldr * a.sign_bytes;
          const int off = grp * SBYTES;
          if constexpr (SEXACT) {
#pragma unroll
            for (int i = 0; i < SBYTES / 4; ++i) reinterpret_cast<uint32_t *>(rec + off)[i] = sw[t][i];
          } else {
            store_bytes<SW>(rec + off, sw[t], min(SBYTES, a.sign_bytes - off));
            if (grp == 3 && 4 * SBYTES < a.sign_bytes) zero_bytes(rec + 4 * SBYTES, a.sign_bytes - 4 * SBYTES);
          }
          if (grp == 0) a.rnorms[vi[t] * a.ldr] = nu[t] > 0.f ? sqrtf(rs[t]) : 0.f;
        }
      }
    }
  }
}

// Kernel arguments of one quantize job (vector i goes to record i * ldr).
inline QArgs make_qargs(const tq_ctx *ctx, const void *x, int64_t n, int64_t ldx, int64_t ldr,
                        uint8_t *codes, uint8_t *signs, float *norms, float *rnorms) {
  QArgs a{};
  a.x = x;
  a.n = n;
  a.ldx = ldx;
  a.ldr = ldr;
  a.codes = codes;
  a.signs = signs;
  a.norms = norms;
  a.rnorms = rnorms;
  a.PiA_hi = ctx->PiA_hi;
  a.PiA_lo = ctx->PiA_lo;
  a.S2A_hi = ctx->S2A_hi;
  a.S2A_lo = ctx->S2A_lo;
  a.d = ctx->hp.d;
  a.m = ctx->hp.m;
  a.prod = ctx->hp.mode == TQ_MODE_PROD;
  a.code_bytes = ctx->code_bytes;
  a.sign_bytes = ctx->sign_bytes;
  for (int j = 0; j < 8; ++j) {
    a.tpos[j] = ctx->tpos[j];
    a.cpos[j] = ctx->cpos[j];
  }
  return a;
}

}  // namespace
}  // namespace tq
