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
#include <cfloat>

#include "tq_score_core.h"

namespace tq {
namespace {

constexpr int CH = 512;            // tokens per chunk
constexpr int NT = 256;            // threads per partial block
constexpr int VB_MAX = 64;         // value code bytes per token handled (d <= 128 at 4 bits; 170 at 3)

struct AttArgs {
  const uint8_t *kcodes, *ksigns;
  const float *knorms, *krnorms;
  const uint8_t *vcodes;
  const float *vnorms;
  const uint8_t *prep;
  float *logits;                   // optional [G][qpg][T]
  float *part;                     // [G*hg][nchunk][4][d + 2]
  int64_t T, ldk;
  int qpg, hg, nchunk, d, kcb, ksb, vcb, vw;
  float alpha, scale;
  float vc[16];                    // value centroids
};

template <int CB16, int SB16, int W>
__global__ void __launch_bounds__(NT) attend_partial_kernel(AttArgs a) {
  constexpr int NM = ScoreShape<CB16, SB16, W>::NM;
  __shared__ __align__(16) float zt[CH][4];         // scaled logits, then weights, [token][head]
  __shared__ __align__(16) uint8_t vbytes[CH * VB_MAX + 16];
  __shared__ float vnu[CH];
  __shared__ float lut[16];
  __shared__ float red[4][NT / 64];
  __shared__ float stat[4][2];
  __shared__ float accs[NT / 64][4][128];          // per-wave partials (d <= 128)

  const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, grp = lane >> 4, wv = tid >> 6;
  const int64_t gidx = blockIdx.y, kg = gidx / a.hg;
  const int hgi = (int)(gidx - kg * a.hg);
  const int chunk = blockIdx.x;
  const int64_t tbeg = (int64_t)chunk * CH;
  const int nval = (int)min((int64_t)CH, a.T - tbeg);
  const int d = a.d;

  // ---- A: logits of this chunk
  {
    const uint8_t *prep = a.prep + gidx * prep_stride(NM);
    i32x4 A[NM];
#pragma unroll
    for (int mu = 0; mu < NM; ++mu) A[mu] = reinterpret_cast<const i32x4 *>(prep)[mu * 64 + lane];
    const float *cst = reinterpret_cast<const float *>(prep + NM * 1024) + grp * 4;
    const HeadConsts hc{cst[0], cst[1], cst[2], cst[3]};
    const int head = hgi * 4 + grp;
    const uint8_t *cb = a.kcodes + kg * a.ldk * a.kcb;
    const uint8_t *sb = a.ksigns + kg * a.ldk * a.ksb;
    const float *nb = a.knorms + kg * a.ldk, *rb = a.krnorms + kg * a.ldk;
    for (int tile = wv; tile * 64 < nval; tile += NT / 64) {
      KeyWords<CB16, SB16, W> kw[4];
      float nu[4], ga[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        int64_t t = tbeg + tile * 64 + 16 * s + col;
        if (t >= a.T) t = a.T - 1;
        load_key_words<true>(kw[s], cb + t * a.kcb, sb + t * a.ksb, grp);
        nu[s] = nb[t];
        ga[s] = rb[t];
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int tl = tile * 64 + 16 * s + col;
        float l = tile_logit<CB16, SB16, W>(A, kw[s], nu[s], ga[s], a.alpha, hc);
        __asm__ volatile("" : "+v"(l));     // keep the norm loads ahead of the guarded stores
        if (tl < nval) {
          zt[tl][grp] = a.scale * l;
          if (a.logits && head < a.qpg) a.logits[(kg * a.qpg + head) * a.T + tbeg + tl] = l;
        }
      }
    }
  }
  // stage value codes and norms of the chunk: batches of independent 16-byte
  // loads from clamped rows (rows past the cache end are never read back)
  {
    const int n16 = CH * a.vcb / 16;                    // multiple of NT (vcb % 16 == 0, CH = 2 NT)
    const uint4 *src = reinterpret_cast<const uint4 *>(a.vcodes + (kg * a.ldk + tbeg) * a.vcb);
    const int lim = nval * a.vcb / 16 - 1;              // last valid 16-byte unit
    for (int base = 0; base < n16; base += 4 * NT) {
      uint4 v[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src) + min(base + b * NT + tid, lim));
        v[b] = make_uint4(t.x, t.y, t.z, t.w);
      }
      // unconditional stores: an index past the end rewrites the last unit
      // with the value it already gets (both loads clamp to the same source)
#pragma unroll
      for (int b = 0; b < 4; ++b) reinterpret_cast<uint4 *>(vbytes)[min(base + b * NT + tid, n16 - 1)] = v[b];
    }
    const float *vn = a.vnorms + kg * a.ldk + tbeg;
    float nv[CH / NT];
#pragma unroll
    for (int b = 0; b < CH / NT; ++b) nv[b] = vn[min(b * NT + tid, nval - 1)];
#pragma unroll
    for (int b = 0; b < CH / NT; ++b) vnu[b * NT + tid] = (b * NT + tid < nval) ? nv[b] : 0.f;
    if (tid < 16) lut[tid] = a.vc[tid & 15];
  }
  for (int t = nval + tid; t < CH; t += NT)
    for (int h = 0; h < 4; ++h) zt[t][h] = -INFINITY;
  for (int i = tid; i < (NT / 64) * 4 * 128; i += NT) (&accs[0][0][0])[i] = 0.f;
  __syncthreads();

  // ---- B: chunk softmax statistics, weights
  float mloc[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  for (int t = tid; t < nval; t += NT)
    for (int h = 0; h < 4; ++h) mloc[h] = fmaxf(mloc[h], zt[t][h]);
  for (int h = 0; h < 4; ++h) {
    float v = mloc[h];
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    if (lane == 0) red[h][wv] = v;
  }
  __syncthreads();
  if (tid < 4) {
    float v = red[tid][0];
    for (int i = 1; i < NT / 64; ++i) v = fmaxf(v, red[tid][i]);
    stat[tid][0] = v;
  }
  __syncthreads();
  float sloc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int t = tid; t < CH; t += NT) {
    for (int h = 0; h < 4; ++h) {
      const float p = t < nval ? __expf(zt[t][h] - stat[h][0]) : 0.f;
      sloc[h] += p;
      zt[t][h] = p * vnu[t];
    }
  }
  for (int h = 0; h < 4; ++h) {
    float v = sloc[h];
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if (lane == 0) red[h][wv] = v;
  }
  __syncthreads();
  if (tid < 4) {
    float v = 0.f;
    for (int i = 0; i < NT / 64; ++i) v += red[tid][i];
    stat[tid][1] = v;
  }

  // ---- C: value accumulation in rotated coordinates
  const int lpt = d / 8;                     // lanes per token (8 coordinates each)
  const int spw = min(64 / lpt, 4);          // token streams per wave (<= 16 per block)
  const int stream = lane / lpt, j = lane - stream * lpt;
  const bool active = stream < spw;
  const int nstreams = spw * (NT / 64);
  const int sid = wv * spw + stream;
  float acc[4][8];
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  if (active) {
    const int vw = a.vw, boff = j * vw;       // this lane's byte run in a record
    const int dw0 = boff >> 2, sh = 8 * (boff & 3);
    const uint32_t mask = (1u << vw) - 1u;
    for (int t = sid; t < nval; t += nstreams) {
      const uint32_t *rec = reinterpret_cast<const uint32_t *>(vbytes + t * a.vcb);
      const uint32_t bits = __builtin_amdgcn_alignbit(rec[dw0 + 1], rec[dw0], sh);
      const float4 wq = *reinterpret_cast<const float4 *>(&zt[t][0]);
      const float w0 = wq.x, w1 = wq.y, w2 = wq.z, w3 = wq.w;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float c = lut[(bits >> (e * vw)) & mask];
        acc[0][e] = fmaf(w0, c, acc[0][e]);
        acc[1][e] = fmaf(w1, c, acc[1][e]);
        acc[2][e] = fmaf(w2, c, acc[2][e]);
        acc[3][e] = fmaf(w3, c, acc[3][e]);
      }
    }
  }
  __syncthreads();
  // ---- D: sum the token streams (lane groups by shuffles, waves via LDS)
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
  float *out = a.part + (gidx * a.nchunk + chunk) * 4 * (d + 2);
  for (int i = tid; i < 4 * d; i += NT) {
    const int h = i / d, c = i - h * d;
    float v = 0.f;
#pragma unroll
    for (int s = 0; s < NT / 64; ++s) v += accs[s][h][c];
    out[h * (d + 2) + c] = v;
  }
  if (tid < 4) {
    out[tid * (d + 2) + d] = stat[tid][0];
    out[tid * (d + 2) + d + 1] = stat[tid][1];
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

int dispatch(const AttArgs &a, dim3 grid, int cb16, int sb16, int w, hipStream_t s) {
#define TQ_CASE(C, S, W_)                                         \
  if (cb16 == C && sb16 == S && w == W_) {                        \
    attend_partial_kernel<C, S, W_><<<grid, NT, 0, s>>>(a);       \
    return hip_status();                                          \
  }
  TQ_FOR_EACH_GEOMETRY(TQ_CASE)
#undef TQ_CASE
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

int launch_attend(const tq_ctx *kc, const tq_ctx *vc, const float *q, int64_t G, int qpg, int64_t T,
                  int64_t ldk, const uint8_t *kcodes, const uint8_t *ksigns, const float *knorms,
                  const float *krnorms, const uint8_t *vcodes, const float *vnorms, float scale,
                  float *logits, float *probs, float *out, void *ws, hipStream_t stream) {
  const int d = kc->hp.d;
  if (d > 128 || d % 16 != 0) return TQ_ENOTSUP;       // value path: 8 coordinates per lane
  if (vc->code_bytes > VB_MAX || (vc->code_bytes * CH) % 16 != 0) return TQ_ENOTSUP;
  if (probs && !logits) return TQ_EINVAL;
  const int hg = (qpg + 3) / 4;
  const int cb16 = kc->code_bytes / 16, sb16 = kc->sign_bytes / 16, w = kc->hp.w;
  const int nm = mfma_count(cb16, sb16, w);
  const int64_t nchunk = (T + CH - 1) / CH;
  const int64_t groups = G * hg;
  if (groups > 65535 || nchunk > MAXCH_LDS || G * qpg > 0x7fffffff) return TQ_ENOTSUP;
  uint8_t *base = reinterpret_cast<uint8_t *>(ws);
  uint8_t *prep = base;
  float *part = reinterpret_cast<float *>(base + align256(groups * prep_stride(nm)));
  float *mstat = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(part) +
                                           align256(groups * nchunk * 4 * (d + 2) * 4));
  int st = launch_prep(kc, q, groups, qpg, hg, G * qpg, prep, stream);
  if (st != TQ_OK) return st;
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
  a.d = d;
  a.kcb = kc->code_bytes;
  a.ksb = kc->sign_bytes;
  a.vcb = vc->code_bytes;
  a.vw = vc->hp.w;
  a.alpha = kc->alpha;
  a.scale = scale;
  for (int i = 0; i < 16; ++i) a.vc[i] = vc->cf[i];
  st = dispatch(a, dim3((unsigned)nchunk, (unsigned)groups), cb16, sb16, w, stream);
  if (st != TQ_OK) return st;
  CombArgs c{};
  c.part = part;
  c.Piv = vc->Pi32;
  c.out = out;
  c.mstat = probs ? mstat : nullptr;
  c.G = G;
  c.qpg = qpg;
  c.hg = hg;
  c.nchunk = (int)nchunk;
  c.d = d;
  attend_combine_kernel<<<(unsigned)(G * qpg), CT, 0, stream>>>(c);
  if (hip_status() != TQ_OK) return TQ_EHIP;
  if (probs) {
    const int64_t rows = G * qpg;
    if (rows > 65535) return TQ_ENOTSUP;
    const unsigned gx = (unsigned)((T + 256 * 8 - 1) / (256 * 8));
    attend_probs_kernel<<<dim3(gx, (unsigned)rows), 256, 0, stream>>>(logits, mstat, probs, T, scale);
    return hip_status();
  }
  return TQ_OK;
}

}  // namespace tq
