// Host-side construction of a context's data-oblivious parameters (float64).
//
// Nothing here looks at data: (d, bits, seed, mode) fixes everything
// (xujun.org note 189244, section 常见问题: data-oblivious, no calibration).
//
//  * Random numbers: SplitMix64 (Steele, Lea, Flood, OOPSLA 2014) in counter
//    form, sub-stream k starting from state seed ^ ((k+1) * golden-gamma),
//    turned into N(0,1) draws by the Box-Muller transform (cosine branch).
//  * Rotation: Householder QR of a d x d Gaussian matrix G (sub-stream 0,
//    row-major), Pi = Q diag(sign R_ii): the Haar-distributed orthogonal
//    matrix the method multiplies every vector by (suzuke blog
//    "turboquant-compressing-ai-consciousness", 技術上怎麼做到的 / 第一步).
//  * JL matrix: S, m x d iid N(0,1) (sub-stream 1), m = d (xujun.org note
//    189244, 第二步：QJL).
//  * Codebook: Max-Lloyd quantizer for N(0,1) with 2^w levels (suzuke blog,
//    第二步), symmetrised, scaled by 1/sqrt(d) for the N(0, 1/d) law of a
//    rotated coordinate (suzuke blog, 第一步).
#include "tq_internal.h"

#include <cmath>
#include <cstring>

namespace tq {

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// count N(0,1) draws of sub-stream `stream` into out[0..count)
void normals(uint64_t seed, int stream, size_t count, double *out) {
  const uint64_t s0 = seed ^ ((uint64_t)(stream + 1) * kGamma);
  const double two_pi = 6.283185307179586476925286766559;
  for (size_t k = 0; k < count; ++k) {
    const uint64_t a = mix64(s0 + (uint64_t)(2 * k + 1) * kGamma);
    const uint64_t b = mix64(s0 + (uint64_t)(2 * k + 2) * kGamma);
    const double u1 = ((double)(a >> 11) + 1.0) * 0x1.0p-53;   // (0, 1]
    const double u2 = (double)(b >> 11) * 0x1.0p-53;           // [0, 1)
    out[k] = std::sqrt(-2.0 * std::log(u1)) * std::cos(two_pi * u2);
  }
}

// In-place Householder QR of A (n x n, row-major).  On return Q (row-major)
// holds the orthogonal factor and rdiag the diagonal of R.
void householder_qr(int n, std::vector<double> &A, std::vector<double> &Q,
                    std::vector<double> &rdiag) {
  std::vector<double> V((size_t)n * n, 0.0);   // reflector k stored in row k
  rdiag.assign(n, 0.0);
  for (int k = 0; k < n; ++k) {
    double norm2 = 0.0;
    for (int i = k; i < n; ++i) norm2 += A[(size_t)i * n + k] * A[(size_t)i * n + k];
    const double norm = std::sqrt(norm2);
    const double x0 = A[(size_t)k * n + k];
    const double alpha = (x0 >= 0.0) ? -norm : norm;      // avoid cancellation
    double *v = &V[(size_t)k * n];
    for (int i = k; i < n; ++i) v[i] = A[(size_t)i * n + k];
    v[k] -= alpha;
    double vn2 = 0.0;
    for (int i = k; i < n; ++i) vn2 += v[i] * v[i];
    if (vn2 > 0.0) {
      const double inv = 1.0 / std::sqrt(vn2);
      for (int i = k; i < n; ++i) v[i] *= inv;
      // A[k:, k:] -= 2 v (v^T A[k:, k:])
      for (int j = k; j < n; ++j) {
        double dot = 0.0;
        for (int i = k; i < n; ++i) dot += v[i] * A[(size_t)i * n + j];
        dot *= 2.0;
        for (int i = k; i < n; ++i) A[(size_t)i * n + j] -= dot * v[i];
      }
    }
    rdiag[k] = A[(size_t)k * n + k];
  }
  // Q = H_0 H_1 ... H_{n-1}: apply the reflectors right-to-left to I.
  Q.assign((size_t)n * n, 0.0);
  for (int i = 0; i < n; ++i) Q[(size_t)i * n + i] = 1.0;
  for (int k = n - 1; k >= 0; --k) {
    const double *v = &V[(size_t)k * n];
    for (int j = 0; j < n; ++j) {
      double dot = 0.0;
      for (int i = k; i < n; ++i) dot += v[i] * Q[(size_t)i * n + j];
      dot *= 2.0;
      for (int i = k; i < n; ++i) Q[(size_t)i * n + j] -= dot * v[i];
    }
  }
}

double phi(double x) {
  if (std::isinf(x)) return 0.0;
  return 0.39894228040143267793994605993438 * std::exp(-0.5 * x * x);
}
double Phi(double x) {
  if (std::isinf(x)) return x > 0 ? 1.0 : 0.0;
  return 0.5 * std::erfc(-x * 0.70710678118654752440084436210485);
}

// Gauss-Legendre rule of n nodes on [-1, 1] (Newton iteration on P_n from
// the Tricomi initial guesses).
void gauss_legendre(int n, std::vector<double> &x, std::vector<double> &w) {
  x.assign(n, 0.0);
  w.assign(n, 0.0);
  const double pi = 3.14159265358979323846264338327950288;
  for (int i = 0; i < n; ++i) {
    double z = std::cos(pi * (i + 0.75) / (n + 0.5)), dp = 1.0;
    for (int it = 0; it < 100; ++it) {
      double p0 = 1.0, p1 = z;
      for (int k = 2; k <= n; ++k) {
        const double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
        p0 = p1;
        p1 = p2;
      }
      dp = n * (z * p1 - p0) / (z * z - 1.0);
      const double dz = p1 / dp;
      z -= dz;
      if (std::fabs(dz) < 1e-16) break;
    }
    x[i] = z;
    w[i] = 2.0 / ((1.0 - z * z) * dp * dp);
  }
}

}  // namespace

// Lloyd-Max quantizer with L levels for the angle of a level-l node of the
// recursive polar transform (l >= 2): the two child radii are lengths of
// independent k-dimensional Gaussian vectors, k = 2^(l-1), so sin^2(phi) is
// Beta(k/2, k/2) and phi has density 2 sin^(k-1) cos^(k-1) / B(k/2, k/2) on
// [0, pi/2] (xujun.org note 189244, 第一步：PolarQuant: the angle laws are
// known and concentrated; suzuke blog, 第二步: a Max-Lloyd codebook per
// angle).  Cells are integrated by a 64-node Gauss-Legendre rule; the
// iteration starts from evenly spaced centroids and the result is made
// symmetric about pi/4.
void lloyd_max_polar_angle(int level, int L, std::vector<double> &c, std::vector<double> &t) {
  static std::vector<double> gx, gw;
  if (gx.empty()) gauss_legendre(64, gx, gw);
  const double half_pi = 1.57079632679489661923132169163975144;
  const double k = std::ldexp(1.0, level - 1);
  const double logB = 2.0 * std::lgamma(0.5 * k) - std::lgamma(k);
  auto dens = [&](double ph) {
    const double sn = std::sin(ph), cs = std::cos(ph);
    if (!(sn > 0.0) || !(cs > 0.0)) return 0.0;
    return 2.0 * std::exp((k - 1.0) * (std::log(sn) + std::log(cs)) - logB);
  };
  c.resize(L);
  for (int i = 0; i < L; ++i) c[i] = (i + 0.5) * half_pi / L;
  std::vector<double> edge(L + 1), next(L);
  for (int it = 0; it < 100000; ++it) {
    edge[0] = 0.0;
    edge[L] = half_pi;
    for (int i = 1; i < L; ++i) edge[i] = 0.5 * (c[i - 1] + c[i]);
    double delta = 0.0;
    for (int i = 0; i < L; ++i) {
      const double a = edge[i], b = edge[i + 1], hw = 0.5 * (b - a), mid = 0.5 * (b + a);
      double m0 = 0.0, m1 = 0.0;
      for (size_t q = 0; q < gx.size(); ++q) {
        const double ph = hw * gx[q] + mid, f = dens(ph) * gw[q];
        m0 += f;
        m1 += f * ph;
      }
      next[i] = m0 > 0.0 ? m1 / m0 : mid;
      delta = std::fmax(delta, std::fabs(next[i] - c[i]));
    }
    c.swap(next);
    if (delta < 1e-14) break;
  }
  for (int i = 0; i < L / 2; ++i) {            // symmetric about pi/4
    const double a = 0.5 * (c[i] + (half_pi - c[L - 1 - i]));
    c[i] = a;
    c[L - 1 - i] = half_pi - a;
  }
  t.resize(L - 1);
  for (int i = 0; i + 1 < L; ++i) t[i] = 0.5 * (c[i] + c[i + 1]);
  if (L % 2 == 0) t[L / 2 - 1] = 0.5 * half_pi;
}

void lloyd_max_unit_gaussian(int L, std::vector<double> &c, std::vector<double> &t) {
  // Alternate the nearest-neighbour condition (thresholds at midpoints) and
  // the centroid condition (each output level is the conditional mean of its
  // cell) from an evenly spaced start until the levels stop moving.
  c.resize(L);
  for (int k = 0; k < L; ++k) c[k] = 3.0 * (2.0 * k + 1.0 - L) / L;
  std::vector<double> edge(L + 1), next(L);
  for (int it = 0; it < 400000; ++it) {
    edge[0] = -INFINITY;
    edge[L] = INFINITY;
    for (int k = 1; k < L; ++k) edge[k] = 0.5 * (c[k - 1] + c[k]);
    double delta = 0.0;
    for (int k = 0; k < L; ++k) {
      next[k] = (phi(edge[k]) - phi(edge[k + 1])) / (Phi(edge[k + 1]) - Phi(edge[k]));
      delta = std::fmax(delta, std::fabs(next[k] - c[k]));
    }
    c.swap(next);
    if (delta < 1e-15) break;
  }
  for (int k = 0; k < L / 2; ++k) {          // exact antisymmetry
    const double a = 0.5 * (c[L - 1 - k] - c[k]);
    c[k] = -a;
    c[L - 1 - k] = a;
  }
  t.resize(L - 1);
  for (int k = 0; k + 1 < L; ++k) t[k] = 0.5 * (c[k] + c[k + 1]);
  t[L / 2 - 1] = 0.0;
}

int build_host_params(int d, int bits, uint64_t seed, int mode, HostParams &hp) {
  if (d < 8 || d > TQ_MAX_D || d % 8 != 0) return TQ_EINVAL;
  if (mode == TQ_MODE_POLAR) {
    // d a power of two of at least 32 (four lane groups of at least 8
    // coordinates each own a subtree of the recursive transform)
    if (d < 32 || d > 256 || (d & (d - 1)) != 0 || bits < 1 || bits > 4) return TQ_EINVAL;
    hp.w = bits;
    hp.m = 0;
  } else if (mode == TQ_MODE_PROD) {
    if (bits < 2 || bits > 4) return TQ_EINVAL;
    hp.w = bits - 1;
    hp.m = d;
  } else if (mode == TQ_MODE_MSE) {
    if (bits < 1 || bits > 4) return TQ_EINVAL;
    hp.w = bits;
    hp.m = 0;
  } else if (mode == TQ_MODE_FRAC) {
    // bits = twice the bits per coordinate; quarters of d/4 coordinates are
    // whole 32-bit plane words
    if ((bits != 5 && bits != 7) || (d != 128 && d != 256)) return TQ_EINVAL;
    hp.w = (bits + 1) / 2 - 1;
    hp.w2 = bits / 2 - 1;
    hp.m = d;
  } else {
    return TQ_EINVAL;
  }
  hp.d = d;
  hp.bits = bits;
  hp.mode = mode;
  hp.seed = seed;
  hp.levels = 1 << hp.w;

  std::vector<double> G((size_t)d * d), Q, rdiag;
  normals(seed, 0, G.size(), G.data());
  householder_qr(d, G, Q, rdiag);
  hp.Pi.resize((size_t)d * d);
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j)
      hp.Pi[(size_t)i * d + j] = Q[(size_t)i * d + j] * (rdiag[j] >= 0.0 ? 1.0 : -1.0);

  hp.S.assign((size_t)hp.m * d, 0.0);
  if (hp.m) normals(seed, 1, hp.S.size(), hp.S.data());

  std::vector<double> c, t;
  if (mode == TQ_MODE_POLAR) {
    // per level l = 1..log2 d: level 1 uniform on [0, 2 pi) (cells of width
    // 2 pi / 2^bits, centroids at their middles), levels >= 2 Lloyd-Max
    const int nl = (int)std::lround(std::log2((double)d)), n = hp.levels;
    const double two_pi = 6.283185307179586476925286766559;
    hp.c.assign((size_t)nl * n, 0.0);
    hp.t.assign((size_t)nl * (n - 1), 0.0);
    for (int i = 0; i < n; ++i) hp.c[i] = (i + 0.5) * two_pi / n;
    for (int i = 1; i < n; ++i) hp.t[i - 1] = i * two_pi / n;
    for (int level = 2; level <= nl; ++level) {
      lloyd_max_polar_angle(level, n, c, t);
      for (int i = 0; i < n; ++i) hp.c[(size_t)(level - 1) * n + i] = c[i];
      for (int i = 0; i + 1 < n; ++i) hp.t[(size_t)(level - 1) * (n - 1) + i] = t[i];
    }
    return TQ_OK;
  }
  lloyd_max_unit_gaussian(hp.levels, c, t);
  const double s = 1.0 / std::sqrt((double)d);
  hp.c.resize(c.size());
  hp.t.resize(t.size());
  for (size_t k = 0; k < c.size(); ++k) hp.c[k] = c[k] * s;
  for (size_t k = 0; k < t.size(); ++k) hp.t[k] = t[k] * s;
  if (mode == TQ_MODE_FRAC) {
    lloyd_max_unit_gaussian(1 << hp.w2, c, t);
    hp.c2.resize(c.size());
    hp.t2.resize(t.size());
    for (size_t k = 0; k < c.size(); ++k) hp.c2[k] = c[k] * s;
    for (size_t k = 0; k < t.size(); ++k) hp.t2[k] = t[k] * s;
  }
  return TQ_OK;
}

}  // namespace tq

extern "C" int tq_host_params(int d, int bits, uint64_t seed, int mode, double *Pi, double *S,
                              double *c, double *t) {
  // prod and MSE-only contexts (a PolarQuant context's codebooks come from
  // tq_polar_codebook: their size differs)
  if (mode != TQ_MODE_PROD && mode != TQ_MODE_MSE && mode != TQ_MODE_FRAC) return TQ_EINVAL;
  tq::HostParams hp;
  const int st = tq::build_host_params(d, bits, seed, mode, hp);
  if (st != TQ_OK) return st;
  if (Pi) std::memcpy(Pi, hp.Pi.data(), hp.Pi.size() * sizeof(double));
  if (S && hp.m) std::memcpy(S, hp.S.data(), hp.S.size() * sizeof(double));
  if (c) {
    std::memcpy(c, hp.c.data(), hp.c.size() * sizeof(double));
    if (!hp.c2.empty()) std::memcpy(c + hp.c.size(), hp.c2.data(), hp.c2.size() * sizeof(double));
  }
  if (t) {
    std::memcpy(t, hp.t.data(), hp.t.size() * sizeof(double));
    if (!hp.t2.empty()) std::memcpy(t + hp.t.size(), hp.t2.data(), hp.t2.size() * sizeof(double));
  }
  return TQ_OK;
}
