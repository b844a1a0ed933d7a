// PolarQuant encoder: the recursive polar transform of the rotated vector,
// every angle coded with its level's Lloyd-Max codebook (xujun.org note
// 189244, section 第一步：PolarQuant: after the random rotation, coordinates
// are paired into (radius, angle), the radii are paired again, recursively,
// down to one radius and a set of angles whose laws are known; suzuke blog
// "turboquant-compressing-ai-consciousness", 技術上怎麼做到的 / 第二步:
// Max-Lloyd points for each angle).
//
//   nu = |x|,  y = Pi x / nu;
//   level 1:   theta_i = atan2(y_{2i+1}, y_{2i}) in [0, 2 pi), r_i = |(y_{2i}, y_{2i+1})|;
//   level l:   phi_j = atan2(r_{2j+1}, r_{2j}) in [0, pi/2], r'_j = |(r_{2j}, r_{2j+1})|;
//   code = number of thresholds of the angle's level strictly below it.
//
// The rotation runs on v_mfma_f32_16x16x32_bf16 exactly as GEMM 1 of the
// quantize kernel (same hi/lo operand fragments and row permutation), so
// lane group g holds the contiguous coordinates [g d/4, (g+1) d/4) of its
// vector: the levels inside that quarter (the quarter's subtree) are
// lane-local, and the last two levels combine the four quarter radii with
// cross-lane reads.  Record slots (b bits each, little-endian): lane group g
// writes slots [g d/4, (g+1) d/4): its subtree's angles level by level, then
// a spare slot that holds the top angle (g = 0), the level L-1 angle of
// quarters 0/1 (g = 1) or of quarters 2/3 (g = 2), or nothing (g = 3).
#include "tq_quantize_body.h"

namespace tq {
namespace {

struct PolarArgs {
  const void *x;
  int64_t n, ldx, ldr, ntiles;
  uint8_t *codes;
  float *norms;
  const Frag *PiA_hi, *PiA_lo;
  const float *thr;        // [level][2^b - 1] thresholds of levels 1..L (level 1 unused)
  int code_bytes;
};

template <int DPAD>
__host__ __device__ constexpr int log2c() {
  int l = 0;
  while ((1 << l) < DPAD) ++l;
  return l;
}

template <int DPAD, bool BF16IN, int B>
__global__ void __launch_bounds__(256) polar_quantize_kernel(PolarArgs a) {
  constexpr int NT = DPAD / 16, NK = DPAD / 32, PER = DPAD / 4;
  constexpr int L = log2c<DPAD>(), LQ = L - 2;    // levels in all, levels inside a quarter
  constexpr int NC = 1 << B;                      // codes per angle
  constexpr int CW = (PER * B + 31) / 32;         // code words per lane
  constexpr int CBYTES = PER * B / 8;             // code bytes per lane (PER >= 8)
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  const float two_pi = 6.28318530717958647692f;

  for (int64_t tile = wave; tile < a.ntiles; tile += nwaves) {
    const int64_t vi = tile * 16 + col;
    const bool valid = vi < a.n;
    // the vector's inputs (bf16 exact, or fp32 as bf16 hi + lo) and its
    // squared length in fp64
    bf16x8 bx[NK], bxl[BF16IN ? 1 : NK];
    double ss = 0.0;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int j0 = k * 32 + grp * 8;
      if constexpr (BF16IN) {
        Frag f = {{0u, 0u, 0u, 0u}};
        if (valid) f = *reinterpret_cast<const Frag *>(reinterpret_cast<const uint16_t *>(a.x) + vi * a.ldx + j0);
        bx[k] = as_bf(f);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double v = (double)(float)bx[k][e];
          ss += v * v;
        }
      } else {
        float xs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (valid) {
          const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.x) + vi * a.ldx + j0);
          const float4 lo4 = p[0], hi4 = p[1];
          xs[0] = lo4.x; xs[1] = lo4.y; xs[2] = lo4.z; xs[3] = lo4.w;
          xs[4] = hi4.x; xs[5] = hi4.y; xs[6] = hi4.z; xs[7] = hi4.w;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += (double)xs[e] * (double)xs[e];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const __bf16 h = (__bf16)xs[e];
          bx[k][e] = h;
          bxl[k][e] = (__bf16)(xs[e] - (float)h);
        }
      }
    }
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    // vectors shorter than 2^-64 are rotated as x * 2^64 (exact), so that no
    // product of the rotation is a float32 denormal
    const bool tiny = ss > 0.0 && ss < 0x1.0p-128;
    const float xsc = tiny ? 0x1.0p64f : 1.f;
    if (__builtin_amdgcn_ballot_w64(tiny) != 0) {
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        if constexpr (BF16IN) {
#pragma unroll
          for (int e = 0; e < 8; ++e) bx[k][e] = (__bf16)((float)bx[k][e] * xsc);
        } else {
          const int j0 = k * 32 + grp * 8;
          float xs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
          if (valid) {
            const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.x) + vi * a.ldx + j0);
            const float4 lo4 = p[0], hi4 = p[1];
            xs[0] = lo4.x; xs[1] = lo4.y; xs[2] = lo4.z; xs[3] = lo4.w;
            xs[4] = hi4.x; xs[5] = hi4.y; xs[6] = hi4.z; xs[7] = hi4.w;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float v = xs[e] * xsc;
            const __bf16 h = (__bf16)v;
            bx[k][e] = h;
            bxl[k][e] = (__bf16)(v - (float)h);
          }
        }
      }
    }
    const double nud = sqrt(ss);
    const float nu = (float)nud;
    const float inv = nud > 0.0 ? (float)(1.0 / (nud * (double)xsc)) : 0.f;

    // y = Pi x / nu: the lane's PER coordinates, 4 per 16-row output tile
    float y[PER];
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        const bf16x8 ah = as_bf(a.PiA_hi[(u * NK + k) * 64 + lane]);
        const bf16x8 al = as_bf(a.PiA_lo[(u * NK + k) * 64 + lane]);
        acc = mfma(ah, bx[k], acc);
        acc = mfma(al, bx[k], acc);
        if constexpr (!BF16IN) acc = mfma(ah, bxl[k], acc);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) y[4 * u + jj] = acc[jj] * inv;
    }

    uint32_t cw[CW];
#pragma unroll
    for (int i = 0; i < CW; ++i) cw[i] = 0u;
    auto put = [&](int slot, uint32_t code) {
      const int bit = slot * B;
      cw[bit >> 5] |= code << (bit & 31);
      if ((bit & 31) + B > 32) cw[(bit >> 5) + 1] |= code >> (32 - (bit & 31));
    };
    // code of a level-l (l >= 2) angle: thresholds strictly below it
    auto code_of = [&](int level, float phi) {
      const float *t = a.thr + (level - 1) * (NC - 1);
      uint32_t c = 0;
#pragma unroll
      for (int k = 0; k < NC - 1; ++k) c += t[k] < phi ? 1u : 0u;
      return c;
    };
    // level 1: angles over the full circle, uniform cells of width 2 pi / NC;
    // an angle exactly on a cell boundary takes the lower cell
    float r[PER / 2];
#pragma unroll
    for (int i = 0; i < PER / 2; ++i) {
      const float ya = y[2 * i], yb = y[2 * i + 1];
      float th = atan2f(yb, ya);
      if (th < 0.f) th += two_pi;
      int c = (int)ceilf(th * ((float)NC / two_pi)) - 1;
      c = c < 0 ? 0 : (c > NC - 1 ? NC - 1 : c);
      put(i, (uint32_t)c);
      r[i] = sqrtf(ya * ya + yb * yb);
    }
    // levels 2 .. L-2 inside the quarter: pairs of radii, in place
    int slot = PER / 2;
#pragma unroll
    for (int level = 2; level <= LQ; ++level) {
#pragma unroll
      for (int i = 0; i < (PER >> level); ++i) {
        const float ra = r[2 * i], rb = r[2 * i + 1];
        put(slot + i, code_of(level, atan2f(rb, ra)));
        r[i] = sqrtf(ra * ra + rb * rb);
      }
      slot += PER >> level;
    }
    // the last two levels, over the four quarter radii of this vector
    const float R0 = __shfl(r[0], col), R1 = __shfl(r[0], col + 16);
    const float R2 = __shfl(r[0], col + 32), R3 = __shfl(r[0], col + 48);
    uint32_t spare = 0u;
    if (grp == 0) spare = code_of(L, atan2f(sqrtf(R2 * R2 + R3 * R3), sqrtf(R0 * R0 + R1 * R1)));
    else if (grp == 1) spare = code_of(L - 1, atan2f(R1, R0));
    else if (grp == 2) spare = code_of(L - 1, atan2f(R3, R2));
    put(PER - 1, spare);
    if (!(nu > 0.f)) {                                    // a zero vector stores zero codes
#pragma unroll
      for (int i = 0; i < CW; ++i) cw[i] = 0u;
    }
    if (valid) {
      uint8_t *rec = a.codes + vi * a.ldr * a.code_bytes;
      const int off = grp * CBYTES;
      store_bytes<CW>(rec + off, cw, CBYTES);
      if (grp == 3 && 4 * CBYTES < a.code_bytes) zero_bytes(rec + 4 * CBYTES, a.code_bytes - 4 * CBYTES);
      if (grp == 0) a.norms[vi * a.ldr] = nu;
    }
  }
}

template <int DPAD, bool BF16IN>
int launch_b(const PolarArgs &a, int b, int blocks, hipStream_t s) {
  switch (b) {
    case 1: polar_quantize_kernel<DPAD, BF16IN, 1><<<blocks, 256, 0, s>>>(a); break;
    case 2: polar_quantize_kernel<DPAD, BF16IN, 2><<<blocks, 256, 0, s>>>(a); break;
    case 3: polar_quantize_kernel<DPAD, BF16IN, 3><<<blocks, 256, 0, s>>>(a); break;
    case 4: polar_quantize_kernel<DPAD, BF16IN, 4><<<blocks, 256, 0, s>>>(a); break;
    default: return TQ_ENOTSUP;
  }
  return hip_status();
}

}  // namespace

int launch_polar_quantize(const tq_ctx *ctx, const void *x, int dtype, int64_t n, int64_t ldx, int64_t ldr,
                          uint8_t *codes, float *norms, hipStream_t stream) {
  if (n == 0) return TQ_OK;
  PolarArgs a{};
  a.x = x;
  a.n = n;
  a.ldx = ldx;
  a.ldr = ldr;
  a.ntiles = (n + 15) / 16;
  a.codes = codes;
  a.norms = norms;
  a.PiA_hi = ctx->PiA_hi;
  a.PiA_lo = ctx->PiA_lo;
  a.thr = ctx->polar_thr;
  a.code_bytes = ctx->code_bytes;
  const int64_t want = (a.ntiles + 3) / 4;          // 4 waves per block, one 16-vector tile each
  const int64_t cap = (int64_t)ctx->cus * 8;
  const int blocks = (int)(want < cap ? (want > 0 ? want : 1) : cap);
  const bool bf16 = dtype == TQ_BF16;
  const int b = ctx->hp.w;
  switch (ctx->hp.d) {
    case 32: return bf16 ? launch_b<32, true>(a, b, blocks, stream) : launch_b<32, false>(a, b, blocks, stream);
    case 64: return bf16 ? launch_b<64, true>(a, b, blocks, stream) : launch_b<64, false>(a, b, blocks, stream);
    case 128: return bf16 ? launch_b<128, true>(a, b, blocks, stream) : launch_b<128, false>(a, b, blocks, stream);
    case 256: return bf16 ? launch_b<256, true>(a, b, blocks, stream) : launch_b<256, false>(a, b, blocks, stream);
    default: return TQ_ENOTSUP;
  }
}

}  // namespace tq
