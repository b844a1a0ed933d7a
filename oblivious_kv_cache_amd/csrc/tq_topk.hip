// Inner-product top-k over a packed database (vector search; xujun.org note
// 189244, section 常见问题: recall 1@k on GloVe d=200).
//
// The estimator of tq_scores.hip is evaluated for every (query, database
// vector) pair, but logits are never written out (at 10^4 x 10^6 they would
// be 40 GB).  Two kernels:
//   scan:  a wave owns 4 queries (one int8-MFMA row group) and one database
//          chunk; every lane keeps a sorted top-KP list (score desc, id asc)
//          of the database vectors it scored, in registers; a new score enters
//          only if it beats the lane's current KP-th best.  The waves of a
//          block scan the same chunk in step, so database lines are reused
//          from the CU's caches.
//   merge: per query, the union of all lane lists (which contains the exact
//          top-k of the GPU scores) is sorted in LDS and the first k are kept.
#include <cfloat>
#include <climits>

#include "tq_score_core.h"

namespace tq {
namespace {

constexpr int MAX_CHUNKS = 8;
// waves (query groups) per scan block: 8 with 16-entry lane lists; 4 with
// 64-entry lists, which need the full register file of one wave per SIMD
__host__ __device__ constexpr int scan_waves(int kp) { return kp <= 16 ? 8 : 4; }

struct TopkGeom {
  int64_t groups;      // query groups of 4
  int64_t qblocks;     // scan blocks along the query axis
  int nchunk;          // database chunks
  int64_t chunk;       // vectors per chunk (multiple of 64)
  int kp;              // per-lane list length (16 or 64)
  int64_t ncand;       // candidates per query
};

TopkGeom topk_geom(int64_t nq, int64_t n, int k) {
  TopkGeom g{};
  g.groups = (nq + 3) / 4;
  g.kp = k <= 16 ? 16 : 64;
  g.qblocks = (g.groups + scan_waves(g.kp) - 1) / scan_waves(g.kp);
  int64_t want = (2048 + g.qblocks - 1) / g.qblocks;
  const int64_t tiles = (n + 63) / 64;
  if (want > tiles) want = tiles;
  if (want > MAX_CHUNKS) want = MAX_CHUNKS;
  if (want < 1) want = 1;
  g.nchunk = (int)want;
  g.chunk = (tiles + g.nchunk - 1) / g.nchunk * 64;
  g.ncand = (int64_t)g.nchunk * 16 * g.kp;
  return g;
}

struct ScanArgs {
  const uint8_t *codes, *signs;
  const float *norms, *rnorms;
  const uint8_t *prep;
  float *cand_s;
  int *cand_i;
  int64_t n, nq, groups, chunk;
  int nchunk, cb, sb, k;
  float alpha;
};

__device__ __forceinline__ bool better(float s, int i, float ts, int ti) {
  return s > ts || (s == ts && i < ti);
}

// k-th largest (k in [1, 16]) of the 16 values held by the lanes of each
// 16-lane row: bitonic sort of the row into descending lane order, then a
// read of lane k - 1.  Every lane of the row gets the result.
__device__ __forceinline__ float row_kth_largest(float v, int k, int lane) {
  const int col = lane & 15;
#pragma unroll
  for (int size = 2; size <= 16; size <<= 1) {
#pragma unroll
    for (int j = size >> 1; j > 0; j >>= 1) {
      const float o = __shfl_xor(v, j);
      const bool desc = (col & size) == 0, lower = (col & j) == 0;
      v = (lower == desc) ? fmaxf(v, o) : fminf(v, o);
    }
  }
  return __shfl(v, (lane & ~15) + k - 1);
}

template <int CB16, int SB16, int W, int KP>
__global__ void __launch_bounds__(64 * scan_waves(KP)) topk_scan_kernel(ScanArgs a) {
  constexpr int NM = ScoreShape<CB16, SB16, W>::NM;
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const int64_t qg = (int64_t)blockIdx.y * scan_waves(KP) + (threadIdx.x >> 6);
  if (qg >= a.groups) return;                      // no block-wide sync below
  const int c = blockIdx.x;
  const uint8_t *prep = a.prep + qg * prep_stride(NM);
  i32x4 A[NM];
#pragma unroll
  for (int mu = 0; mu < NM; ++mu) A[mu] = reinterpret_cast<const i32x4 *>(prep)[mu * 64 + lane];
  const float *cst = reinterpret_cast<const float *>(prep + NM * 1024) + grp * 4;
  const HeadConsts hc = HeadConsts::load(cst);
  const ParityMasks<CB16, W> pm = parity_masks<CB16, W>(grp);

  float ls[KP];
  int li[KP];
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    ls[j] = -FLT_MAX;
    li[j] = INT_MAX;
  }
  // n < 2^31 and record offsets < 2^32 are checked on the host
  const int begin = (int)((int64_t)c * a.chunk);
  const int end = (int)min((int64_t)begin + a.chunk, a.n);
  // Pruning bound for k <= 16: the k-th largest of the 16 lanes' current
  // best scores of a query.  k distinct vectors score at least that much, so
  // a score below it cannot be in the query's top k; refreshed every 4 tiles.
  float thr = -FLT_MAX;
  int tile = 0;
  for (int t0 = begin; t0 < end; t0 += 64, ++tile) {
    KeyWords<CB16, SB16, W> kw[4];
    float nu[4], ga[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t t = (uint32_t)min(t0 + 16 * s + col, end - 1);
      load_key_words<false>(kw[s], a.codes, a.signs, t, grp);
      nu[s] = load_f32(a.norms, t);
      ga[s] = load_f32(a.rnorms, t);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int t = t0 + 16 * s + col;
      const float l = tile_logit<CB16, SB16, W>(A, kw[s], nu[s], ga[s], a.alpha, hc, pm);
      const bool want = t < end && l > ls[KP - 1] && !(l < thr);
      // few scores pass once the lists have filled: a wave-uniform branch
      // skips the insertion network
      if (__builtin_amdgcn_ballot_w64(want) == 0) continue;
      if (want) {
        // ids seen by a lane increase, so a tie with the last entry never enters
        float cs = l;
        int ci = t;
#pragma unroll
        for (int j = 0; j < KP; ++j) {
          const bool b = better(cs, ci, ls[j], li[j]);
          const float ts = ls[j];
          const int ti = li[j];
          ls[j] = b ? cs : ts;
          li[j] = b ? ci : ti;
          cs = b ? ts : cs;
          ci = b ? ti : ci;
        }
      }
    }
    if (a.k <= 16 && (tile & 3) == 3) thr = row_kth_largest(ls[0], a.k, lane);
  }
  const int64_t q = qg * 4 + grp;
  if (q < a.nq) {
    const int64_t base = ((q * a.nchunk + c) * 16 + col) * KP;
#pragma unroll
    for (int j = 0; j < KP; ++j) {
      a.cand_s[base + j] = ls[j];
      a.cand_i[base + j] = li[j];
    }
  }
}

// Sort each query's candidates by (score desc, id asc) in LDS; keep the first k.
__global__ void __launch_bounds__(256) topk_merge_kernel(const float *cand_s, const int *cand_i,
                                                         int64_t ncand, int npow2, int k,
                                                         int64_t *ids, float *scores) {
  extern __shared__ unsigned char smem[];
  float *ss = reinterpret_cast<float *>(smem);
  int *si = reinterpret_cast<int *>(ss + npow2);
  const int64_t q = blockIdx.x;
  for (int i = threadIdx.x; i < npow2; i += 256) {
    if (i < ncand) {
      ss[i] = cand_s[q * ncand + i];
      si[i] = cand_i[q * ncand + i];
    } else {
      ss[i] = -FLT_MAX;
      si[i] = INT_MAX;
    }
  }
  __syncthreads();
  // bitonic sort, "better" first
  for (int size = 2; size <= npow2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < npow2 / 2; i += 256) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = ((lo & size) == 0);
        const float s0 = ss[lo], s1 = ss[hi];
        const int i0 = si[lo], i1 = si[hi];
        const bool swap = desc ? better(s1, i1, s0, i0) : better(s0, i0, s1, i1);
        if (swap) {
          ss[lo] = s1; ss[hi] = s0;
          si[lo] = i1; si[hi] = i0;
        }
      }
      __syncthreads();
    }
  }
  for (int j = threadIdx.x; j < k; j += 256) {
    ids[q * k + j] = si[j];
    scores[q * k + j] = ss[j];
  }
}

int dispatch_scan(const ScanArgs &a, dim3 grid, int cb16, int sb16, int w, int kp, hipStream_t s) {
#define TQ_CASE(C, S, W_)                                                              \
  if (cb16 == C && sb16 == S && w == W_) {                                             \
    if (kp == 16)                                                                      \
      topk_scan_kernel<C, S, W_, 16><<<grid, 64 * scan_waves(16), 0, s>>>(a);          \
    else                                                                               \
      topk_scan_kernel<C, S, W_, 64><<<grid, 64 * scan_waves(64), 0, s>>>(a);          \
    return hip_status();                                                               \
  }
  TQ_FOR_EACH_GEOMETRY(TQ_CASE)
#undef TQ_CASE
  return TQ_ENOTSUP;
}

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t topk_ws_bytes(const tq_ctx *ctx, int64_t nq, int64_t n, int k) {
  const TopkGeom g = topk_geom(nq, n, k);
  const int nm = mfma_count(ctx->code_bytes / 16, ctx->sign_bytes / 16, ctx->hp.w);
  return (size_t)(align256(g.groups * prep_stride(nm)) + 2 * align256(nq * g.ncand * 4));
}

int launch_topk(const tq_ctx *ctx, const float *q, int64_t nq, int64_t n, const uint8_t *codes,
                const uint8_t *signs, const float *norms, const float *rnorms, int k,
                int64_t *ids, float *scores, void *ws, hipStream_t stream) {
  const TopkGeom g = topk_geom(nq, n, k);
  const int cb16 = ctx->code_bytes / 16, sb16 = ctx->sign_bytes / 16, w = ctx->hp.w;
  const int nm = mfma_count(cb16, sb16, w);
  uint8_t *base = reinterpret_cast<uint8_t *>(ws);
  uint8_t *prep = base;
  float *cand_s = reinterpret_cast<float *>(base + align256(g.groups * prep_stride(nm)));
  int *cand_i = reinterpret_cast<int *>(reinterpret_cast<uint8_t *>(cand_s) + align256(nq * g.ncand * 4));
  if (n > INT_MAX || g.qblocks > 65535 || nq > 0x7fffffff) return TQ_ENOTSUP;
  // record offsets are 32-bit in the scan kernel
  if (n * (int64_t)(ctx->code_bytes > ctx->sign_bytes ? ctx->code_bytes : ctx->sign_bytes) >= ((int64_t)1 << 32))
    return TQ_ENOTSUP;
  int st = launch_prep(ctx, q, g.groups, 4, 1, nq, prep, stream);
  if (st != TQ_OK) return st;
  ScanArgs a{};
  a.codes = codes;
  a.signs = signs;
  a.norms = norms;
  a.rnorms = rnorms;
  a.prep = prep;
  a.cand_s = cand_s;
  a.cand_i = cand_i;
  a.n = n;
  a.nq = nq;
  a.groups = g.groups;
  a.chunk = g.chunk;
  a.nchunk = g.nchunk;
  a.cb = ctx->code_bytes;
  a.sb = ctx->sign_bytes;
  a.alpha = ctx->alpha;
  a.k = k;
  st = dispatch_scan(a, dim3((unsigned)g.nchunk, (unsigned)g.qblocks), cb16, sb16, w, g.kp, stream);
  if (st != TQ_OK) return st;
  int npow2 = 1;
  while (npow2 < g.ncand) npow2 <<= 1;
  const size_t lds = (size_t)npow2 * 8;
  topk_merge_kernel<<<(unsigned)nq, 256, lds, stream>>>(cand_s, cand_i, g.ncand, npow2, k, ids, scores);
  return hip_status();
}

}  // namespace tq
