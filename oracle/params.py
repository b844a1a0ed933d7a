"""Data-oblivious parameters: rotation, JL matrix, Lloyd-Max codebook (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

* Rotation: a random orthogonal matrix applied to every vector (suzuke blog,
  "技術上怎麼做到的 / 第一步"; xujun.org note 189244, "第一步：PolarQuant").
  Built as the QR factor of a Gaussian matrix with the signs of R's diagonal
  moved into Q, which makes it Haar-distributed (Mezzadri, "How to generate
  random matrices from the classical compact groups", 2007).
* JL matrix S: m x d with iid N(0,1) entries, m = d (xujun.org note 189244,
  "第二步：QJL").
* Codebook: Max-Lloyd scalar quantizer (suzuke blog, "第二步": best
  quantization points by the Max-Lloyd algorithm) for the law of a rotated
  unit-vector coordinate, read as N(0, 1/d) (suzuke blog, "第一步").  The
  codebook is built for N(0,1) and scaled by 1/sqrt(d).
"""

import math
from dataclasses import dataclass
from statistics import NormalDist

import numpy as np

from .rng import gaussian_stream

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def haar_rotation(d, seed):
    """Pi = Q diag(sign R_ii) for G = QR, G[d x d] row-major from stream 0."""
    g = gaussian_stream(seed, 0, d * d).reshape(d, d)
    q, r = np.linalg.qr(g)
    return q * np.sign(np.diag(r))[None, :]


def jl_matrix(d, m, seed):
    """S [m x d], iid N(0,1), row-major from stream 1 (no orthogonalisation)."""
    return gaussian_stream(seed, 1, m * d).reshape(m, d)


def _phi(x):
    if math.isinf(x):
        return 0.0
    return _INV_SQRT_2PI * math.exp(-0.5 * x * x)


def _Phi(x):
    if x == math.inf:
        return 1.0
    if x == -math.inf:
        return 0.0
    return 0.5 * math.erfc(-x / _SQRT2)


def lloyd_max_gaussian(levels, tol=1e-15, max_iter=200000):
    """Lloyd-Max quantizer for N(0,1) with ``levels`` output points.

    Alternates the two optimality conditions until the centroids move by less
    than ``tol``: thresholds at midpoints of adjacent centroids, and each
    centroid equal to the conditional mean of its cell,
        c_k = (phi(t_{k-1}) - phi(t_k)) / (Phi(t_k) - Phi(t_{k-1})).
    Starts from the quantiles (k + 1/2)/L.  The result is symmetrised
    (c_{L-1-k} = -c_k, middle threshold exactly 0).

    Returns (centroids ascending [L], thresholds ascending [L-1]) for N(0,1).
    """
    L = int(levels)
    if L < 2:
        raise ValueError("need at least 2 levels")
    nd = NormalDist()
    c = [nd.inv_cdf((k + 0.5) / L) for k in range(L)]
    for _ in range(max_iter):
        t = [-math.inf] + [(c[k] + c[k + 1]) / 2.0 for k in range(L - 1)] + [math.inf]
        new = []
        for k in range(L):
            mass = _Phi(t[k + 1]) - _Phi(t[k])
            new.append((_phi(t[k]) - _phi(t[k + 1])) / mass)
        delta = max(abs(a - b) for a, b in zip(new, c))
        c = new
        if delta < tol:
            break
    c = np.array(c, dtype=np.float64)
    c = 0.5 * (c - c[::-1])
    t = 0.5 * (c[:-1] + c[1:])
    if L % 2 == 0:
        t[L // 2 - 1] = 0.0
    return c, t


def gaussian_distortion(c, t):
    """E[(g - Q(g))^2] for g ~ N(0,1) and a centroid-condition codebook.

    With each centroid at its cell's conditional mean the distortion is
    1 - sum_k c_k^2 P(cell k) (textbook identity for Lloyd-Max quantizers).
    """
    edges = [-math.inf] + [float(x) for x in t] + [math.inf]
    tot = 1.0
    for k, ck in enumerate(c):
        tot -= ck * ck * (_Phi(edges[k + 1]) - _Phi(edges[k]))
    return tot


def codebook(d, code_bits):
    """Centroids and thresholds for N(0, 1/d) at ``code_bits`` bits."""
    c, t = lloyd_max_gaussian(2 ** code_bits)
    s = 1.0 / math.sqrt(d)
    return c * s, t * s


@dataclass
class TQParams:
    """All data-oblivious state for one (d, bits, seed, mode)."""

    d: int
    bits: int
    seed: int
    mode: str          # "prod": (bits-1)-bit codes + 1-bit QJL; "mse": bits-bit codes
    m: int             # JL rows (= d in prod mode, 0 in mse mode)
    w: int             # code bits per coordinate
    Pi: np.ndarray     # [d, d]
    S: np.ndarray      # [m, d] (empty in mse mode)
    c: np.ndarray      # [2^w] ascending centroids for N(0, 1/d)
    t: np.ndarray      # [2^w - 1] ascending thresholds

    @property
    def alpha(self):
        """Residual-correction scale sqrt(pi/2)/m.

        Not printed on the pages; it is the unique constant that makes the
        estimator unbiased (xujun.org note 189244, "第二步：QJL": the estimate
        equals the true inner product in expectation): for s ~ N(0, I),
        E[sign(<s, v>) <s, q>] = sqrt(2/pi) <v, q> / |v|.
        """
        return math.sqrt(math.pi / 2.0) / self.m


def make_params(d, bits, seed, mode="prod"):
    """Build the parameters of one context.

    prod mode: bits in {2,3,4}; code bits w = bits - 1; m = d (suzuke blog,
    "第二步": b-1 bits for the codebook stage, "第三步": the last bit for QJL).
    mse mode: bits in {1,2,3,4}; w = bits; no JL matrix.
    """
    if d < 8 or d % 8 != 0:
        raise ValueError("d must be a positive multiple of 8")
    if mode == "prod":
        if bits not in (2, 3, 4):
            raise ValueError("prod mode needs bits in {2,3,4}")
        w, m = bits - 1, d
    elif mode == "mse":
        if bits not in (1, 2, 3, 4):
            raise ValueError("mse mode needs bits in {1,2,3,4}")
        w, m = bits, 0
    else:
        raise ValueError(mode)
    Pi = haar_rotation(d, seed)
    S = jl_matrix(d, m, seed) if m else np.zeros((0, d))
    c, t = codebook(d, w)
    return TQParams(d=d, bits=bits, seed=seed, mode=mode, m=m, w=w, Pi=Pi, S=S, c=c, t=t)
