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
//   partial kernel (block = one chunk of one query group):
//     A. int8-MFMA logits of the chunk into LDS (and to the optional logits
//        output);
//     B. chunk max m and sum l of exp(z - m) per head, weights
//        w_t = exp(z_t - m) nu_t in LDS;
//     C. value codes of the chunk staged in LDS with 16-byte loads; lanes own
//        8 rotated coordinates (one record byte run each), token streams
//        split across lane groups and waves; centroids from an LDS table;
//     D. stream partials summed through LDS; (m, l, acc[d]) written out.
//   combine kernel: merges chunks with the usual max rescaling, divides by
//     the total, applies Pi_v^T; optionally normalises the logits to probs.
#include <algorithm>
#include <cfloat>

#include "tq_score_core.h"

namespace tq {
namespace {

constexpr int CH = 512;            // tokens per chunk
constexpr int NT = 256;            // threads per partial block
constexpr int VB_MAX = 64;         // value code bytes per token handled (d <= 128 at 4 bits; 170 at 3)
#ifndef TQ_ATT_BLOCKS
#define TQ_ATT_BLOCKS 512          // partial blocks per call (2 per CU are resident)
#endif

struct AttArgs {
  const uint8_t *kcodes, *ksigns;
  const float *knorms, *krnorms;
  const uint8_t *vcodes;
  const float *vnorms;
  const uint8_t *prep;
  float *logits;                   // optional [G][qpg][T]
  float *part;                     // [G*hg][nsplit][4][d + 2]
  int64_t T, ldk;
  int qpg, hg, nchunk, nsplit, cps, d, kcb, ksb, vcb, vw;
  float alpha, scale;
  float vc[16];                    // value centroids
};

// One block = one query group x one split (a run of `cps` chunks of CH
// tokens), with an online softmax over the chunks: the running max M and the
// value accumulators (rotated coordinates, in registers) are rescaled by
// exp(M_old - M_new) whenever a chunk raises the max.  The key words, value
// codes and value norms of chunk c+1 are loaded into registers while chunk c
// is processed, so every block keeps its next ~50 KB in flight.
#ifndef TQ_ATT_WAVES_PER_EU
#define TQ_ATT_WAVES_PER_EU 2
#endif
template <int CB16, int SB16, int W, int VR>      // VR = value code bytes / 8 = 16-byte units per thread per chunk
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(TQ_ATT_WAVES_PER_EU)))
attend_partial_kernel(AttArgs a) {
  constexpr int NM = ScoreShape<CB16, SB16, W>::NM;
  using KW = KeyWords<CB16, SB16, W>;
  __shared__ __align__(16) float zt[CH][4];         // scaled logits, then weights, [token][head]
  __shared__ __align__(16) uint8_t vbytes[CH * VB_MAX + 16];
  __shared__ float vnu[CH];
  __shared__ float2 lut2[256];                       // (c[a], c[b]) for the code pair a | b << vw
  __shared__ float red[4][NT / 64];
  __shared__ float accs[NT / 64][4][128];          // per-wave partials (d <= 128)

  const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, grp = lane >> 4, wv = tid >> 6;
  const int64_t gidx = blockIdx.y, kg = gidx / a.hg;
  const int hgi = (int)(gidx - kg * a.hg);
  const int c_begin = blockIdx.x * a.cps;
  const int c_end = min(c_begin + a.cps, a.nchunk);
  const int d = a.d;
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
  const uint8_t *vcb = a.vcodes + kg * a.ldk * a.vcb;
  const float *vnb = a.vnorms + kg * a.ldk;
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

  {
    const int vw = a.vw, np = 1 << (2 * vw);
    __shared__ float lut[16];
    if (tid < 16) lut[tid] = a.vc[tid & 15];
    __syncthreads();
    for (int i = tid; i < np; i += NT) lut2[i] = make_float2(lut[i & ((1 << vw) - 1)], lut[i >> vw]);
  }
  for (int i = tid; i < (NT / 64) * 4 * 128; i += NT) (&accs[0][0][0])[i] = 0.f;

  // registers of the chunk in flight: key words per 16-key subtile; key norms
  // one per lane (lane l: key l of each of the wave's two 64-key tiles),
  // handed to the lanes that need them by cross-lane reads
  KW kw[2][4];
  float knu[2], kga[2];
  u32x4 vr[VR];
  float vn[CH / NT];
  auto issue = [&](int c) {
    // 32-bit offsets from the group's base pointers (the host checks that a
    // group's records span less than 4 GB) keep the address math short
    const int tbeg = c * CH, tlast = (int)T - 1;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t t = (uint32_t)min(tbeg + (wv + 4 * tt) * 64 + 16 * s + col, tlast);
        const uint8_t *cp = kcb + (t * (CB16 * 16) + (uint32_t)grp * (CB16 * 4));
        const uint8_t *sp = ksb + (t * (SB16 * 16) + (uint32_t)grp * (SB16 * 4));
#pragma unroll
        for (int i = 0; i < CB16; ++i) kw[tt][s].cw[i] = key_word<true>(reinterpret_cast<const uint32_t *>(cp + 4 * i));
#pragma unroll
        for (int i = 0; i < SB16; ++i) kw[tt][s].sw[i] = key_word<true>(reinterpret_cast<const uint32_t *>(sp + 4 * i));
      }
      const uint32_t tl = (uint32_t)min(tbeg + (wv + 4 * tt) * 64 + lane, tlast);
      knu[tt] = load_f32(knb, tl);
      kga[tt] = load_f32(krb, tl);
    }
    // value codes: clamped 16-byte units (units past the cache end repeat the
    // last real one and are never read back)
    const uint32_t lim = (uint32_t)(min(CH, (int)T - tbeg) * (VR / 2)) - 1u;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(vcb + (uint32_t)tbeg * (VR * 8));
#pragma unroll
    for (int b = 0; b < VR; ++b) vr[b] = __builtin_nontemporal_load(src + min((uint32_t)(b * NT + tid), lim));
#pragma unroll
    for (int b = 0; b < CH / NT; ++b) vn[b] = vnb[(uint32_t)min(tbeg + b * NT + tid, tlast)];
  };

  // value-stream geometry: lanes own 8 rotated coordinates (one byte run of a
  // record); token streams are split across lane groups and waves
  // (d <= 128: at least 4 streams fit in a wave; 16 streams per block)
  constexpr int SPW = 4, NSTREAM = SPW * (NT / 64);
  const int lpt = d / 8;
  const int stream = lane / lpt, j = lane - stream * lpt;
  const bool active = stream < SPW;
  const int sid = wv * SPW + stream;
  const int vw = a.vw, boff = j * vw;
  const int dw0 = boff >> 2, sh = 8 * (boff & 3);

  float M[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  float lsum[4] = {0.f, 0.f, 0.f, 0.f};
  float acc[4][8];
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

  issue(c_begin);
  for (int c = c_begin; c < c_end; ++c) {
    const int64_t tbeg = (int64_t)c * CH;
    const int nval = (int)min((int64_t)CH, T - tbeg);
    // ---- A: logits of the chunk; value codes and norms to LDS
    // all eight 16-key logits first (independent MFMA chains interleave),
    // then the stores
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
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int tl = (wv + 4 * tt) * 64 + 16 * s + col;
        zt[tl][grp] = tl < nval ? a.scale * lg[tt][s] : -INFINITY;
      }
    if (a.logits && head < a.qpg) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int tl = (wv + 4 * tt) * 64 + 16 * s + col;
          if (tl < nval) a.logits[(kg * a.qpg + head) * T + tbeg + tl] = lg[tt][s];
        }
    }
#pragma unroll
    for (int b = 0; b < VR; ++b)
      reinterpret_cast<u32x4 *>(vbytes)[b * NT + tid] = vr[b];
#pragma unroll
    for (int b = 0; b < CH / NT; ++b) vnu[b * NT + tid] = b * NT + tid < nval ? vn[b] : 0.f;
    if (c + 1 < c_end) issue(c + 1);
    __syncthreads();

    // ---- B: chunk max, new running max, weights w_t = exp(z_t - M) nu_t
    float f[4];
    {
      const float4 z0 = *reinterpret_cast<const float4 *>(&zt[tid][0]);
      const float4 z1 = *reinterpret_cast<const float4 *>(&zt[tid + NT][0]);
      const float mx[4] = {fmaxf(z0.x, z1.x), fmaxf(z0.y, z1.y), fmaxf(z0.z, z1.z), fmaxf(z0.w, z1.w)};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float t = wave_max(mx[h]);
        if (lane == 0) red[h][wv] = t;
      }
      __syncthreads();
      float p0[4], p1[4];
      const float za[4] = {z0.x, z0.y, z0.z, z0.w}, zb[4] = {z1.x, z1.y, z1.z, z1.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        float mc = red[h][0];
#pragma unroll
        for (int i = 1; i < NT / 64; ++i) mc = fmaxf(mc, red[h][i]);
        const float mn = fmaxf(M[h], mc);
        f[h] = M[h] == -INFINITY ? 0.f : __expf(M[h] - mn);
        M[h] = mn;
        p0[h] = __expf(za[h] - mn);
        p1[h] = __expf(zb[h] - mn);
        lsum[h] = fmaf(lsum[h], f[h], p0[h] + p1[h]);
      }
      const float n0 = vnu[tid], n1 = vnu[tid + NT];
      *reinterpret_cast<float4 *>(&zt[tid][0]) = make_float4(p0[0] * n0, p0[1] * n0, p0[2] * n0, p0[3] * n0);
      *reinterpret_cast<float4 *>(&zt[tid + NT][0]) = make_float4(p1[0] * n1, p1[1] * n1, p1[2] * n1, p1[3] * n1);
    }
    __syncthreads();

    // ---- C: rescale the accumulators, add this chunk's weighted centroids
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= f[h];
    if (active) {
      // every token of the chunk: past nval the weights are 0 and the staged
      // codes are copies of real ones; a fixed trip count lets the LDS reads
      // of several tokens be in flight together
#pragma unroll 4
      for (int k = 0; k < CH / NSTREAM; ++k) {
        const int t = sid + NSTREAM * k;
        const uint32_t *rec = reinterpret_cast<const uint32_t *>(vbytes + t * a.vcb);
        const uint32_t bits = __builtin_amdgcn_alignbit(rec[dw0 + 1], rec[dw0], sh);
        const float4 wq = *reinterpret_cast<const float4 *>(&zt[t][0]);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float2 cv = lut2[__builtin_amdgcn_ubfe(bits, e * vw, 2 * vw)];
          acc[0][e] = fmaf(wq.x, cv.x, acc[0][e]);
          acc[1][e] = fmaf(wq.y, cv.x, acc[1][e]);
          acc[2][e] = fmaf(wq.z, cv.x, acc[2][e]);
          acc[3][e] = fmaf(wq.w, cv.x, acc[3][e]);
          acc[0][e + 1] = fmaf(wq.x, cv.y, acc[0][e + 1]);
          acc[1][e + 1] = fmaf(wq.y, cv.y, acc[1][e + 1]);
          acc[2][e + 1] = fmaf(wq.z, cv.y, acc[2][e + 1]);
          acc[3][e + 1] = fmaf(wq.w, cv.y, acc[3][e + 1]);
        }
      }
    }
    __syncthreads();      // zt, vbytes and red are rewritten by the next chunk
  }

  // ---- D: block totals: sums over threads, accumulators over token streams
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const float t = wave_sum(lsum[h]);
    if (lane == 0) red[h][wv] = t;
  }
  const bool by_group = (lpt == 16);          // d == 128: the 4 streams are the 4 lane groups
  if (by_group) {
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = acc[h][e];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        acc[h][e] = v;
      }
  }
  if (active && (!by_group || stream == 0)) {
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (by_group) accs[wv][h][8 * j + e] = acc[h][e];
        else atomicAdd(&accs[wv][h][8 * j + e], acc[h][e]);
      }
  }
  __syncthreads();
  float *out = a.part + (gidx * a.nsplit + blockIdx.x) * 4 * (d + 2);
  for (int i = tid; i < 4 * d; i += NT) {
    const int h = i / d, cc = i - h * d;
    float v = 0.f;
#pragma unroll
    for (int s = 0; s < NT / 64; ++s) v += accs[s][h][cc];
    out[h * (d + 2) + cc] = v;
  }
  if (tid < 4) {
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) l += red[tid][i];
    const float mt = tid == 0 ? M[0] : tid == 1 ? M[1] : tid == 2 ? M[2] : M[3];
    out[tid * (d + 2) + d] = mt;
    out[tid * (d + 2) + d + 1] = l;
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
// code sizes 16, 32, 48, 64 bytes.
int dispatch(const AttArgs &a, dim3 grid, int cb16, int sb16, int w, hipStream_t s) {
  const int vr = a.vcb / 8;
#define TQ_CASE_V(C, S, W_, V)                                         \
  if (vr == V) {                                                       \
    attend_partial_kernel<C, S, W_, V><<<grid, NT, 0, s>>>(a);         \
    return hip_status();                                               \
  }
#define TQ_CASE(C, S, W_)                                              \
  if (cb16 == C && sb16 == S && w == W_) {                             \
    TQ_CASE_V(C, S, W_, 2) TQ_CASE_V(C, S, W_, 4) TQ_CASE_V(C, S, W_, 6) TQ_CASE_V(C, S, W_, 8) \
    return TQ_ENOTSUP;                                                 \
  }
  TQ_CASE(1, 1, 1) TQ_CASE(1, 1, 2) TQ_CASE(2, 1, 2) TQ_CASE(1, 1, 3) TQ_CASE(2, 1, 3) TQ_CASE(3, 1, 3)
#undef TQ_CASE
#undef TQ_CASE_V
  return TQ_ENOTSUP;
}

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t attend_ws_bytes(const tq_ctx *k, int64_t G, int qpg, int64_t T) {
  const int hg = (qpg + 3) / 4;
  const int nm = mfma_count(k->code_bytes / 16, k->sign_bytes / 16, k->hp.w);
  const int64_t nchunk = (T + CH - 1) / CH;
  const int d = k->hp.d;
  return (size_t)(align256(G * hg * prep_stride(nm)) + align256(G * hg * nchunk * 4 * (d + 2) * 4) +
                  align256(G * qpg * 2 * 4));
}

int check_attend(const tq_ctx *kc, const tq_ctx *vc, int64_t G, int qpg, int64_t T, int64_t ldk,
                 bool want_probs) {
  const int d = kc->hp.d;
  if (d > 128 || d % 16 != 0) return TQ_ENOTSUP;       // value path: 8 coordinates per lane
  if (vc->code_bytes > VB_MAX || (vc->code_bytes * CH) % 16 != 0) return TQ_ENOTSUP;
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
  const int cb16 = kc->code_bytes / 16, sb16 = kc->sign_bytes / 16, w = kc->hp.w;
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
  // splits per query group: about TQ_ATT_BLOCKS blocks in all, equal runs of chunks
  int64_t want = (TQ_ATT_BLOCKS + groups - 1) / groups;
  if (want > nchunk) want = nchunk;
  if (want < 1) want = 1;
  a.cps = (int)((nchunk + want - 1) / want);
  a.nsplit = (int)((nchunk + a.cps - 1) / a.cps);
  a.d = d;
  a.kcb = kc->code_bytes;
  a.ksb = kc->sign_bytes;
  a.vcb = vc->code_bytes;
  a.vw = vc->hp.w;
  a.alpha = kc->alpha;
  a.scale = scale;
  for (int i = 0; i < 16; ++i) a.vc[i] = vc->cf[i];
  st = dispatch(a, dim3((unsigned)a.nsplit, (unsigned)groups), cb16, sb16, w, stream);
  if (st != TQ_OK) return st;
  CombArgs c{};
  c.part = part;
  c.Piv = vc->Pi32;
  c.out = out;
  c.mstat = probs ? mstat : nullptr;
  c.G = G;
  c.qpg = qpg;
  c.hg = hg;
  c.nchunk = a.nsplit;
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
