// Inner-product top-k over a packed database (vector search; xujun.org note
// 189244, section 常见问题: recall 1@k on GloVe d=200).
//
// The estimator of tq_scores.hip is evaluated for every (query, database
// vector) pair, but logits are never written out (at 10^4 x 10^6 they would
// be 40 GB).  Two kernels:
//   scan:  a wave owns 4 or 8 queries (one or two int8-MFMA row groups) and
//          one database chunk; every lane keeps a sorted top-KP list (score desc, id asc)
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
// Query groups per scan wave: with 16-entry lists and records of up to 12
// MFMAs per tile, a wave scores two groups against each database tile and
// builds every bit-plane operand once for both (the planes are most of the
// VALU work per MFMA; 2^20-key scans at d=200, b=2: 26.2 -> 22.3 ms).  Larger
// records would not fit two groups' fragments and lists in registers.
__host__ __device__ constexpr int scan_qg(int kp, int nm) { return kp <= 16 && nm <= 12 ? 2 : 1; }

struct TopkGeom {
  int64_t groups;      // query groups of 4
  int64_t qblocks;     // scan blocks along the query axis
  int nchunk;          // database chunks
  int64_t chunk;       // vectors per chunk (multiple of 64)
  int kp;              // per-lane list length (16 or 64)
  int64_t ncand;       // candidates per query
};

TopkGeom topk_geom(int64_t nq, int64_t n, int k, int nm, int cus) {
  TopkGeom g{};
  g.groups = (nq + 3) / 4;
  g.kp = k <= 16 ? 16 : 64;
  const int per_block = scan_waves(g.kp) * scan_qg(g.kp, nm);
  g.qblocks = (g.groups + per_block - 1) / per_block;
  int64_t want = (2048 + g.qblocks - 1) / g.qblocks;
  const int64_t tiles = (n + 63) / 64;
  if (want > tiles) want = tiles;
  if (want > MAX_CHUNKS) want = MAX_CHUNKS;
  if (want < 1) want = 1;
  // A scan block fills its CU (8 waves at two per SIMD, or 4 at one), so the
  // blocks run in rounds of `cus`.  From want up to MAX_CHUNKS chunks, take
  // the count with the fewest rounds per unit of work (the fullest last
  // round; ties: fewer chunks, less to merge).
  int64_t best = want, best_rounds = (g.qblocks * want + cus - 1) / cus;
  for (int64_t nc = want + 1; nc <= MAX_CHUNKS && nc <= tiles; ++nc) {
    const int64_t rounds = (g.qblocks * nc + cus - 1) / cus;
    if (rounds * best < best_rounds * nc) {
      best = nc;
      best_rounds = rounds;
    }
  }
  want = best;
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
  constexpr int QG = scan_qg(KP, NM);
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const int64_t qg0 = ((int64_t)blockIdx.y * scan_waves(KP) + (threadIdx.x >> 6)) * QG;
  if (qg0 >= a.groups) return;                     // no block-wide sync below
  const int c = blockIdx.x;
  // the wave's query groups qg0 .. qg0 + QG - 1 (past the last group, the
  // last one again: scored, never stored)
  i32x4 A[QG][NM];
  HeadConsts hc[QG];
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    const uint8_t *prep = a.prep + min(qg0 + g, a.groups - 1) * prep_stride(NM);
#pragma unroll
    for (int mu = 0; mu < NM; ++mu) A[g][mu] = reinterpret_cast<const i32x4 *>(prep)[mu * 64 + lane];
    hc[g] = HeadConsts::load(reinterpret_cast<const float *>(prep + NM * 1024) + grp * 4);
  }
  const ParityMasks<CB16, W> pm = parity_masks<CB16, W>(grp);

  float ls[QG][KP];
  int li[QG][KP];
#pragma unroll
  for (int g = 0; g < QG; ++g)
#pragma unroll
    for (int j = 0; j < KP; ++j) {
      ls[g][j] = -FLT_MAX;
      li[g][j] = INT_MAX;
    }
  // n < 2^31 and record offsets < 2^32 are checked on the host
  const int begin = (int)((int64_t)c * a.chunk);
  const int end = (int)min((int64_t)begin + a.chunk, a.n);
  // Pruning bound for k <= 16: the k-th largest of the 16 lanes' current
  // best scores of a query.  k distinct vectors score at least that much, so
  // a score below it cannot be in the query's top k; refreshed every 4 tiles.
  float thr[QG];
#pragma unroll
  for (int g = 0; g < QG; ++g) thr[g] = -FLT_MAX;
  // Register set of one 64-key tile: the key words of its four 16-key
  // subtiles, and its norms one per lane (lane l: key t0 + l), handed to the
  // lanes that need them by a cross-lane read; the next lane group's first
  // code word (3-bit codes) also comes from its lane.
  struct Buf {
    KeyWords<CB16, SB16, W> kw[4];
    float nu, ga;
  };
  auto load = [&](Buf &buf, int t0) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t t = (uint32_t)min(t0 + 16 * s + col, end - 1);
      const uint8_t *cp = a.codes + (t * (CB16 * 16) + (uint32_t)grp * (CB16 * 4));
      const uint8_t *sp = a.signs + (t * (SB16 * 16) + (uint32_t)grp * (SB16 * 4));
#pragma unroll
      for (int i = 0; i < CB16; ++i) buf.kw[s].cw[i] = key_word<false>(reinterpret_cast<const uint32_t *>(cp + 4 * i));
#pragma unroll
      for (int i = 0; i < SB16; ++i) buf.kw[s].sw[i] = key_word<false>(reinterpret_cast<const uint32_t *>(sp + 4 * i));
    }
    const uint32_t tl = (uint32_t)min(t0 + lane, end - 1);
    buf.nu = load_f32(a.norms, tl);
    buf.ga = load_f32(a.rnorms, tl);
  };
  auto score = [&](Buf &buf, int t0, int tile) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if constexpr (W == 3) {   // first code word of the next lane group (lane + 16), none for the last
        const uint32_t nxt = (uint32_t)__shfl((int)buf.kw[s].cw[0], (lane + 16) & 63);
        buf.kw[s].cw[CB16] = grp < 3 ? nxt : 0u;
      }
      const float nu = __shfl(buf.nu, 16 * s + col), ga = __shfl(buf.ga, 16 * s + col);
      const int t = t0 + 16 * s + col;
      float lq[QG];
      tile_logits<CB16, SB16, W, QG>(A, buf.kw[s], nu, ga, a.alpha, hc, pm, lq);
#pragma unroll
      for (int g = 0; g < QG; ++g) {
        const float l = lq[g];
        const bool want = t < end && l > ls[g][KP - 1] && !(l < thr[g]);
        // few scores pass once the lists have filled: a wave-uniform branch
        // skips the insertion network
        if (__builtin_amdgcn_ballot_w64(want) == 0) continue;
        if (want) {
          // ids seen by a lane increase, so a tie with the last entry never enters
          float cs = l;
          int ci = t;
#pragma unroll
          for (int j = 0; j < KP; ++j) {
            const bool b = better(cs, ci, ls[g][j], li[g][j]);
            const float ts = ls[g][j];
            const int ti = li[g][j];
            ls[g][j] = b ? cs : ts;
            li[g][j] = b ? ci : ti;
            cs = b ? ts : cs;
            ci = b ? ti : ci;
          }
        }
      }
    }
    if (a.k <= 16 && (tile & 3) == 3) {
#pragma unroll
      for (int g = 0; g < QG; ++g) thr[g] = row_kth_largest(ls[g][0], a.k, lane);
    }
  };
  // (a second register set, to overlap the next tile's loads, measured no
  // faster: the scan is bound by VALU and MFMA issue, not by load latency)
  int tile = 0;
  for (int t0 = begin; t0 < end; t0 += 64, ++tile) {
    Buf buf;
    load(buf, t0);
    score(buf, t0, tile);
  }
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    const int64_t q = (qg0 + g) * 4 + grp;
    if (qg0 + g < a.groups && q < a.nq) {
      const int64_t base = ((q * a.nchunk + c) * 16 + col) * KP;
#pragma unroll
      for (int j = 0; j < KP; ++j) {
        a.cand_s[base + j] = ls[g][j];
        a.cand_i[base + j] = li[g][j];
      }
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

// ---------------------------------------------------------------- large k
// k up to TQ_MAX_TOPK, or records of vectors longer than 256 coordinates:
// one 256-thread block per (query group of 4, database chunk).  The block
// keeps, per query, a sorted list of the best LIST entries seen (in LDS, with
// the group's A fragments) and a candidate buffer.  The four waves score 256
// database vectors per round (big_tiles); a score enters the buffer only if it
// beats the list's k-th entry (vectors of later rounds have larger ids, so a
// tie never enters).  When a buffer may overflow in the next round, the block
// sorts it and merges it into the list.  The chunk's list goes to the
// candidate array that topk_merge_kernel reduces over chunks.
constexpr int LIST = 1024;        // list capacity (>= k)
constexpr int CBUF = 1024;        // candidate buffer per query
constexpr int BLK_ROUND = 256;    // vectors scored per round (4 waves x 64)

struct BlkArgs {
  const uint8_t *codes, *signs;
  const float *norms, *rnorms;
  const uint8_t *prep;
  float *cand_s;
  int *cand_i;
  int64_t n, nq, chunk;
  int nchunk, cb16, sb16, nm, k;
  float alpha;
};

template <int W>
__global__ void __launch_bounds__(256) topk_block_kernel(BlkArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  i32x4 *Al = reinterpret_cast<i32x4 *>(smem);
  float *bs = reinterpret_cast<float *>(Al + a.nm * 64);     // [4][LIST + CBUF]
  int *bi = reinterpret_cast<int *>(bs + 4 * (LIST + CBUF));
  __shared__ int cnt[4];
  __shared__ float thr[4];
  constexpr int ROW = LIST + CBUF;
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, grp = lane >> 4, wv = tid >> 6;
  const int64_t qg = blockIdx.y;
  const int c = blockIdx.x;
  const uint8_t *prep = a.prep + qg * prep_stride(a.nm);
  stage_frags(Al, prep, a.nm, tid, 256);
  for (int i = tid; i < 4 * ROW; i += 256) {
    bs[i] = -FLT_MAX;
    bi[i] = INT_MAX;
  }
  if (tid < 4) {
    cnt[tid] = 0;
    thr[tid] = -FLT_MAX;
  }
  const HeadConsts hc = HeadConsts::load(reinterpret_cast<const float *>(prep + (int64_t)a.nm * 1024) + grp * 4);
  __syncthreads();

  // candidates of every query sorted worst first, then merged into the lists:
  // [list best first | candidates worst first] is bitonic; the better half of
  // each compare-exchange at distance LIST is the best LIST of both, and a
  // bitonic merge sorts it
  auto merge = [&]() {
    for (int size = 2; size <= CBUF; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < 4 * (CBUF / 2); i += 256) {
          const int qq = i / (CBUF / 2), ii = i - qq * (CBUF / 2);
          const int lo = 2 * ii - (ii & (stride - 1)), hi = lo + stride;
          float *rs = bs + qq * ROW + LIST;
          int *ri = bi + qq * ROW + LIST;
          const bool worst_first = (lo & size) == 0;
          const float s0 = rs[lo], s1 = rs[hi];
          const int i0 = ri[lo], i1 = ri[hi];
          const bool swap = worst_first ? better(s0, i0, s1, i1) : better(s1, i1, s0, i0);
          if (swap) {
            rs[lo] = s1; rs[hi] = s0;
            ri[lo] = i1; ri[hi] = i0;
          }
        }
        __syncthreads();
      }
    }
    for (int i = tid; i < 4 * LIST; i += 256) {
      const int qq = i / LIST, ii = i - qq * LIST;
      float *rs = bs + qq * ROW;
      int *ri = bi + qq * ROW;
      const float s0 = rs[ii], s1 = rs[ii + LIST];
      const int i0 = ri[ii], i1 = ri[ii + LIST];
      if (better(s1, i1, s0, i0)) {
        rs[ii] = s1;
        ri[ii] = i1;
      }
      rs[ii + LIST] = -FLT_MAX;          // the buffer is emptied
      ri[ii + LIST] = INT_MAX;
    }
    __syncthreads();
    for (int stride = LIST / 2; stride > 0; stride >>= 1) {
      for (int i = tid; i < 4 * (LIST / 2); i += 256) {
        const int qq = i / (LIST / 2), ii = i - qq * (LIST / 2);
        const int lo = 2 * ii - (ii & (stride - 1)), hi = lo + stride;
        float *rs = bs + qq * ROW;
        int *ri = bi + qq * ROW;
        const float s0 = rs[lo], s1 = rs[hi];
        const int i0 = ri[lo], i1 = ri[hi];
        if (better(s1, i1, s0, i0)) {
          rs[lo] = s1; rs[hi] = s0;
          ri[lo] = i1; ri[hi] = i0;
        }
      }
      __syncthreads();
    }
    if (tid < 4) {
      cnt[tid] = 0;
      // the k-th entry bounds what can still enter (none while the list is short)
      thr[tid] = bi[tid * ROW + a.k - 1] == INT_MAX ? -FLT_MAX : bs[tid * ROW + a.k - 1];
    }
    __syncthreads();
  };

  const int64_t begin = (int64_t)c * a.chunk;
  const int64_t end = min(begin + a.chunk, a.n);
  const int64_t cbytes = 16 * a.cb16, sbytes = 16 * a.sb16;
  const uint8_t *cbase = a.codes + grp * a.cb16 * 4;
  const uint8_t *sbase = a.signs + grp * a.sb16 * 4;
  for (int64_t r0 = begin; r0 < end; r0 += BLK_ROUND) {
    const int64_t t0 = r0 + wv * 64;
    if (t0 < end) {
      const uint8_t *cp[4];
      const uint8_t *sp[4];
      float nu[4], ga[4], l[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int64_t t = min(t0 + 16 * s + col, end - 1);
        cp[s] = cbase + t * cbytes;
        sp[s] = sbase + t * sbytes;
        nu[s] = a.norms[t];
        ga[s] = a.rnorms[t];
      }
      big_tiles<W, 4>(Al, cp, sp, a.cb16, a.sb16, lane, nu, ga, a.alpha, hc, l);
      const float th = thr[grp];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int64_t t = t0 + 16 * s + col;
        if (t < end && l[s] > th) {
          const int pos = atomicAdd(&cnt[grp], 1);
          bs[grp * ROW + LIST + pos] = l[s];
          bi[grp * ROW + LIST + pos] = (int)t;
        }
      }
    }
    __syncthreads();
    const bool last = r0 + BLK_ROUND >= end;
    const int most = max(max(cnt[0], cnt[1]), max(cnt[2], cnt[3]));
    // every thread has read the counters before the next round adds to them,
    // so the decision is the same in all threads
    __syncthreads();
    if (most > CBUF - BLK_ROUND || (last && most > 0)) merge();
  }
  for (int i = tid; i < 4 * a.k; i += 256) {
    const int qq = i / a.k, j = i - qq * a.k;
    const int64_t q = qg * 4 + qq;
    if (q < a.nq) {
      const int64_t o = (q * a.nchunk + c) * a.k + j;
      a.cand_s[o] = bs[qq * ROW + j];
      a.cand_i[o] = bi[qq * ROW + j];
    }
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

// The block path (k > 64, or d > 256): chunks so that about two blocks per CU
// run, at most 8, and at most 8192 candidates per query for the final sort.
bool topk_block_path(const tq_ctx *ctx, int k) { return k > 64 || ctx->hp.d > 256; }

TopkGeom topk_block_geom(const tq_ctx *ctx, int64_t nq, int64_t n, int k) {
  TopkGeom g{};
  g.groups = (nq + 3) / 4;
  g.qblocks = g.groups;
  int64_t want = (2 * (int64_t)ctx->cus + g.groups - 1) / g.groups;
  const int64_t rounds = (n + BLK_ROUND - 1) / BLK_ROUND;
  if (want > rounds) want = rounds;
  if (want > MAX_CHUNKS) want = MAX_CHUNKS;
  if (want * k > 8192) want = 8192 / k;
  if (want < 1) want = 1;
  g.nchunk = (int)want;
  g.chunk = (rounds + want - 1) / want * BLK_ROUND;
  g.nchunk = (int)((n + g.chunk - 1) / g.chunk);
  g.kp = 0;
  g.ncand = (int64_t)g.nchunk * k;
  return g;
}

}  // namespace

size_t topk_ws_bytes(const tq_ctx *ctx, int64_t nq, int64_t n, int k) {
  const int nm = mfma_count(ctx->cw16, ctx->sign_bytes / 16, ctx->hp.w);
  const TopkGeom g = topk_block_path(ctx, k) ? topk_block_geom(ctx, nq, n, k) : topk_geom(nq, n, k, nm, ctx->cus);
  return (size_t)(align256(g.groups * prep_stride(nm)) + 2 * align256(nq * g.ncand * 4));
}

int launch_topk(const tq_ctx *ctx, const float *q, int64_t nq, int64_t n, const uint8_t *codes,
                const uint8_t *signs, const float *norms, const float *rnorms, int k,
                int64_t *ids, float *scores, void *ws, hipStream_t stream) {
  const int cb16 = ctx->cw16, sb16 = ctx->sign_bytes / 16, w = ctx->hp.w;
  const int nm = mfma_count(cb16, sb16, w);
  const bool blk = topk_block_path(ctx, k);
  const TopkGeom g = blk ? topk_block_geom(ctx, nq, n, k) : topk_geom(nq, n, k, nm, ctx->cus);
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
  if (blk) {
    BlkArgs b{};
    b.codes = codes;
    b.signs = signs;
    b.norms = norms;
    b.rnorms = rnorms;
    b.prep = prep;
    b.cand_s = cand_s;
    b.cand_i = cand_i;
    b.n = n;
    b.nq = nq;
    b.chunk = g.chunk;
    b.nchunk = g.nchunk;
    b.cb16 = cb16;
    b.sb16 = sb16;
    b.nm = nm;
    b.k = k;
    b.alpha = ctx->alpha;
    const size_t lds = (size_t)nm * 1024 + 4 * (size_t)(LIST + CBUF) * 8;
    const void *fn = w == 3 ? reinterpret_cast<const void *>(&topk_block_kernel<3>)
                            : reinterpret_cast<const void *>(&topk_block_kernel<1>);
    if ((st = allow_lds(fn, lds)) != TQ_OK) return st;
    const dim3 grid((unsigned)g.nchunk, (unsigned)g.groups);
    if (w == 3)
      topk_block_kernel<3><<<grid, 256, lds, stream>>>(b);
    else
      topk_block_kernel<1><<<grid, 256, lds, stream>>>(b);
    if ((st = hip_status()) != TQ_OK) return st;
  } else {
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
  }
  int npow2 = 1;
  while (npow2 < g.ncand) npow2 <<= 1;
  const size_t lds = (size_t)npow2 * 8;
  topk_merge_kernel<<<(unsigned)nq, 256, lds, stream>>>(cand_s, cand_i, g.ncand, npow2, k, ids, scores);
  return hip_status();
}

}  // namespace tq
