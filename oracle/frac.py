"""Fractional bit widths: 2.5 and 3.5 bits per coordinate (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages report TurboQuant at 2.5 and 3.5 bits per channel (suzuke blog
"turboquant-compressing-ai-consciousness", "實際跑出來的數據": 3.5 bits
matches FP16 on LongBench and 2.5 bits is about 1.2% lower; xujun.org note
189244, "跑分全面碾压": community runs at 2.5 and 3.5 bits), but they print
no mechanism.  The reading taken here is the plainest one that keeps the rest
of the method unchanged:

  * b = B / 2 with B odd: the rotated coordinates fall into two fixed halves.
    Rotated coordinates 0 .. d/2 - 1 take w_hi = ceil(b) - 1 code bits and
    the rest w_lo = floor(b) - 1, each half with the Lloyd-Max codebook for
    N(0, 1/d) at its own width (suzuke blog, "第二步"), so the codes average
    b - 1 bits; the QJL stage is unchanged (one sign bit per JL row, m = d,
    of the stage-1 residual over all coordinates: xujun.org note 189244,
    "第二步：QJL"), for b bits per coordinate in all.
  * The split depends on d alone.  Pi is a Haar rotation, so any fixed split
    of its output coordinates has the same law; the method stays
    data-oblivious, and the estimator keeps its form,
        l = nu ( <Pi q, c_hat> + alpha gamma <S q, 2 bits - 1> ),
    with c_hat_i the centroid of coordinate i in its half's codebook.
  * Record layout (none on the pages; this is the library's): the d
    coordinates form 4 quarters of d/4; quarter g stores w_g bit planes of
    d/4 bits each (w_g = w_hi for g < 2, w_lo after), plane p holding bit p
    of the codes of the quarter's coordinates in order; quarters follow one
    another, LSB first, for code_bytes = d (w_hi + w_lo) / 16 (d a multiple
    of 32; no padding).  Signs, norms and residual norms as for integer
    widths.

Pinned in ``tests/test_oracle_frac.py``.
"""

import math

import numpy as np

from .params import codebook, haar_rotation, jl_matrix
from .quant import record_sizes


class FracParams:
    """Data-oblivious state of one fractional-width context.

    half_bits = 2 b (5 or 7).  ``widths`` overrides (w_hi, w_lo) for tests
    that reduce the scheme to an integer width (w_hi == w_lo)."""

    def __init__(self, d, half_bits, seed, widths=None):
        if d < 32 or d % 32 != 0:
            raise ValueError("fractional widths need d a multiple of 32")
        if widths is None:
            if half_bits not in (5, 7):
                raise ValueError("half_bits in {5, 7} (2.5 or 3.5 bits)")
            widths = ((half_bits + 1) // 2 - 1, half_bits // 2 - 1)
        self.d, self.half_bits, self.seed = d, half_bits, seed
        self.w_hi, self.w_lo = widths
        self.m = d
        self.mode = "prod"
        self.Pi = haar_rotation(d, seed)
        self.S = jl_matrix(d, d, seed)
        self.c_hi, self.t_hi = codebook(d, self.w_hi)
        self.c_lo, self.t_lo = codebook(d, self.w_lo)
        self.code_bytes = d * (self.w_hi + self.w_lo) // 16
        self.sign_bytes = record_sizes(d, 1, d)[1]

    @property
    def alpha(self):
        return math.sqrt(math.pi / 2.0) / self.m

    def hi(self):
        """Boolean mask of the coordinates coded at w_hi bits."""
        return np.arange(self.d) < self.d // 2

    def centroids(self, idx):
        """c_hat [n, d] from per-coordinate indices idx [n, d]."""
        idx = np.asarray(idx)
        out = np.empty(idx.shape, np.float64)
        h = self.d // 2
        out[:, :h] = self.c_hi[idx[:, :h]]
        out[:, h:] = self.c_lo[idx[:, h:]]
        return out


def pack(p, idx):
    """Planar record bytes [n, code_bytes] from code indices idx [n, d]."""
    idx = np.asarray(idx, np.int64)
    n, q = idx.shape[0], p.d // 4
    bits = []
    for g in range(4):
        w = p.w_hi if g < 2 else p.w_lo
        blk = idx[:, g * q:(g + 1) * q]
        for plane in range(w):
            bits.append(((blk >> plane) & 1).astype(np.uint8))
    allbits = np.concatenate(bits, axis=1) if bits else np.zeros((n, 0), np.uint8)
    assert allbits.shape[1] == 8 * p.code_bytes
    return np.packbits(allbits, axis=1, bitorder="little")


def unpack(p, codes):
    """Inverse of :func:`pack`: idx [n, d]."""
    bits = np.unpackbits(np.asarray(codes, np.uint8), axis=1, bitorder="little").astype(np.int64)
    n, q = bits.shape[0], p.d // 4
    idx = np.zeros((n, p.d), np.int64)
    off = 0
    for g in range(4):
        w = p.w_hi if g < 2 else p.w_lo
        for plane in range(w):
            idx[:, g * q:(g + 1) * q] |= bits[:, off:off + q] << plane
            off += q
    return idx


def _codes_of(p, y):
    """idx = #{k : t_k < y_i} in each coordinate's own half (ties take the lower index)."""
    h = p.d // 2
    idx = np.empty(y.shape, np.int64)
    idx[:, :h] = np.searchsorted(p.t_hi, y[:, :h], side="left")
    idx[:, h:] = np.searchsorted(p.t_lo, y[:, h:], side="left")
    return idx


def quantize(p, X, return_unpacked=False):
    """Records (codes, signs, norms, rnorms) of the rows of X, step by step as
    for integer widths: nu = |x|, y = Pi x / nu, per-coordinate codes in the
    coordinate's half, r = y - c_hat, gamma = |r|, bits = [S (x/nu - Pi^T c_hat) >= 0]."""
    X = np.asarray(X).astype(np.float64)
    n = X.shape[0]
    nu = np.sqrt(np.sum(X * X, axis=1))
    zero = nu == 0.0
    u = X / np.where(zero, 1.0, nu)[:, None]
    y = u @ p.Pi.T
    idx = _codes_of(p, y)
    idx[zero] = 0
    chat = p.centroids(idx)
    r = y - chat
    gamma = np.sqrt(np.sum(r * r, axis=1))
    gamma[zero] = 0.0
    z = (u - chat @ p.Pi) @ p.S.T
    sbits = (z >= 0.0).astype(np.int64)
    sbits[zero] = 0
    signs = np.zeros((n, p.sign_bytes * 8), np.uint8)
    signs[:, :p.m] = sbits
    out = {"codes": pack(p, idx), "signs": np.packbits(signs, axis=1, bitorder="little"),
           "norms": nu.astype(np.float32), "rnorms": gamma.astype(np.float32)}
    if return_unpacked:
        out.update(idx=idx, sbits=sbits, y=np.where(zero[:, None], 0.0, y), z=z)
    return out


def stage2_from_codes(p, x, idx):
    """(gamma, z, bits) of one vector for a given code choice idx [d]."""
    x = np.asarray(x, np.float64)
    u = x / np.sqrt(np.sum(x * x))
    y = p.Pi @ u
    chat = p.centroids(np.asarray(idx)[None, :])[0]
    r = y - chat
    z = p.S @ (u - p.Pi.T @ chat)
    return float(np.sqrt(np.sum(r * r))), z, (z >= 0.0).astype(np.int64)


def _sign_values(p, signs):
    bits = np.unpackbits(np.asarray(signs, np.uint8), axis=1, bitorder="little")[:, :p.m]
    return 2.0 * bits.astype(np.float64) - 1.0


def scores(p, Q, codes, signs, norms, rnorms):
    """Logits [nq, n] of queries Q [nq, d] against n records."""
    Q = np.asarray(Q, np.float64)
    chat = p.centroids(unpack(p, codes))
    approx = (Q @ p.Pi.T) @ chat.T
    corr = (Q @ p.S.T) @ _sign_values(p, signs).T
    nu = np.asarray(norms, np.float64)[None, :]
    gamma = np.asarray(rnorms, np.float64)[None, :]
    return nu * (approx + p.alpha * gamma * corr)


def dequant(p, codes, signs, norms, rnorms):
    """x_hat = nu (Pi^T c_hat + alpha gamma S^T (2 bits - 1))."""
    chat = p.centroids(unpack(p, codes))
    xhat = chat @ p.Pi + p.alpha * np.asarray(rnorms, np.float64)[:, None] * (_sign_values(p, signs) @ p.S)
    return np.asarray(norms, np.float64)[:, None] * xhat
