"""PolarQuant: recursive polar coordinates of the rotated vector (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages describe PolarQuant as the stage that does the main compression
(xujun.org note 189244, "第一步：PolarQuant"; suzuke blog, "技術上怎麼做到的 /
第二步"): after the random rotation, coordinates are paired and each pair is
written as (radius, angle); the radii are paired again and the same
transform applied, recursively, until one final radius and a set of angles
remain.  The law of every angle is known and concentrated, so each angle is
coded with a Max-Lloyd quantizer built for that law, and no normalisation
constant is stored.

Readings taken here (the pages give no formulas):
  * d is a power of two, d = 2^L; level 1 pairs coordinates (2i, 2i+1) of
    y = Pi x / |x| and has d/2 angles theta = atan2(y_{2i+1}, y_{2i}) in
    [0, 2 pi); level l >= 2 pairs the radii (2j, 2j+1) of level l-1 and has
    d / 2^l angles phi = atan2(r_{2j+1}, r_{2j}) in [0, pi/2]; the last
    radius is |y| = 1 and is not stored (the length |x| is, as float32);
  * the laws: a rotated unit vector is uniform on the sphere, equivalently a
    normalised Gaussian vector, so theta is uniform on [0, 2 pi), and at
    level l >= 2 the two radii are lengths of independent k-dimensional
    Gaussian vectors, k = 2^(l-1): sin^2(phi) ~ Beta(k/2, k/2), with density
    f_l(phi) = 2 sin^(k-1)(phi) cos^(k-1)(phi) / B(k/2, k/2) on [0, pi/2];
  * every angle takes ``bits`` bits (MSE-only stage; the same budget as the
    scalar codes of tq_init_mse), with the Lloyd-Max quantizer of its level's
    law: at level 1 the uniform quantizer (cells of width 2 pi / 2^bits,
    centroids at their middles), at level >= 2 the Lloyd-Max iteration
    (thresholds at midpoints, centroids at the conditional means, found by
    quadrature of f_l), symmetrised about pi/4;
  * an angle exactly on a threshold takes the lower index (as for the scalar
    codes); atan2(0, 0) = 0;
  * record layout (none on the pages): the d angle-code slots of ``bits``
    bits, little-endian as for the scalar codes, are grouped by quarter of the
    coordinates: slots [q d/4, (q+1) d/4) hold the angles of the subtree over
    coordinates [q d/4, (q+1) d/4), level by level (level 1 first, in pair
    order), then one spare slot; the spare slot of quarter 0 holds the top
    angle (level L), of quarter 1 the level L-1 angle of quarters 0/1, of
    quarter 2 the level L-1 angle of quarters 2/3, of quarter 3 nothing
    (zero).  d = 4 is the smallest case with quarters of one coordinate
    (no level inside a quarter); d must be at least 8 here.
"""

import math

import numpy as np

from .params import haar_rotation
from .quant import pack_bits, unpack_bits, record_sizes

TWO_PI = 2.0 * math.pi


def levels(d):
    """L with d = 2^L (d a power of two, d >= 8)."""
    L = int(round(math.log2(d)))
    if d < 8 or 2 ** L != d:
        raise ValueError("PolarQuant needs d a power of two, d >= 8")
    return L


def angle_density(level, phi):
    """Density of a level-l angle (l >= 2) at phi in [0, pi/2] (array or scalar)."""
    k = 2 ** (level - 1)
    logB = 2.0 * math.lgamma(k / 2.0) - math.lgamma(float(k))
    phi = np.asarray(phi, np.float64)
    s, c = np.sin(phi), np.cos(phi)
    with np.errstate(divide="ignore"):
        logf = (k - 1) * (np.log(s) + np.log(c)) - logB
    return np.where((s > 0.0) & (c > 0.0), 2.0 * np.exp(logf), 0.0 if k > 1 else 2.0 / math.pi)


_GL_X, _GL_W = np.polynomial.legendre.leggauss(64)


def _cell_moments(level, a, b):
    """(mass, first moment) of the level-l angle law on the cells [a_i, b_i]
    (arrays) by 64-node Gauss-Legendre quadrature."""
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    half, mid = 0.5 * (b - a), 0.5 * (b + a)
    phis = half[:, None] * _GL_X[None, :] + mid[:, None]
    f = angle_density(level, phis)
    return half * (f @ _GL_W), half * ((f * phis) @ _GL_W)


def lloyd_max_angle(level, L, tol=1e-14, max_iter=100000):
    """Lloyd-Max quantizer with L levels for the level-l angle law (l >= 2) on
    [0, pi/2]: thresholds at midpoints, centroids at conditional means, from
    equally spaced centroids; symmetrised about pi/4.  Returns (c [L], t [L-1])."""
    lo, hi = 0.0, 0.5 * math.pi
    c = lo + (np.arange(L) + 0.5) * (hi - lo) / L
    for _ in range(max_iter):
        t = np.concatenate([[lo], 0.5 * (c[:-1] + c[1:]), [hi]])
        m0, m1 = _cell_moments(level, t[:-1], t[1:])
        new = np.where(m0 > 0, m1 / np.where(m0 > 0, m0, 1.0), 0.5 * (t[:-1] + t[1:]))
        delta = float(np.max(np.abs(new - c)))
        c = new
        if delta < tol:
            break
    c = 0.5 * (c + (0.5 * math.pi - c[::-1]))          # symmetric about pi/4
    t = 0.5 * (c[:-1] + c[1:])
    if L % 2 == 0:
        t[L // 2 - 1] = 0.25 * math.pi
    return c, t


def codebooks(d, bits):
    """Per level l = 1..L: (centroids, thresholds) of its angles."""
    L = levels(d)
    n = 2 ** bits
    books = [(np.array([(i + 0.5) * TWO_PI / n for i in range(n)]),
              np.array([i * TWO_PI / n for i in range(1, n)]))]
    for level in range(2, L + 1):
        books.append(lloyd_max_angle(level, n))
    return books


def polar_angles(y):
    """Exact recursive polar transform of y [d]: a list of per-level angle
    arrays (level 1 in [0, 2 pi), higher levels in [0, pi/2]) and the final
    radius."""
    y = np.asarray(y, np.float64)
    a, b = y[0::2], y[1::2]
    theta = np.arctan2(b, a)
    theta = np.where(theta < 0.0, theta + TWO_PI, theta)
    r = np.hypot(a, b)
    out = [theta]
    while r.size > 1:
        ra, rb = r[0::2], r[1::2]
        out.append(np.arctan2(rb, ra))
        r = np.hypot(ra, rb)
    return out, float(r[0])


def polar_reconstruct(angles, radius=1.0):
    """Inverse of :func:`polar_angles`: y from per-level angles and the final radius."""
    r = np.array([radius])
    for phi in reversed(angles[1:]):
        child = np.empty(2 * r.size)
        child[0::2] = r * np.cos(phi)
        child[1::2] = r * np.sin(phi)
        r = child
    theta = angles[0]
    y = np.empty(2 * r.size)
    y[0::2] = r * np.cos(theta)
    y[1::2] = r * np.sin(theta)
    return y


def _slot_order(d):
    """For each record slot: (level, index within the level) or None (spare)."""
    L = levels(d)
    P = d // 4                      # coordinates per quarter
    slots = []
    for q in range(4):
        for level in range(1, L - 1):          # levels inside a quarter
            n_q = P >> level                   # angles of this level in the quarter
            for i in range(n_q):
                slots.append((level, q * n_q + i))
        slots.append({0: (L, 0), 1: (L - 1, 0), 2: (L - 1, 1), 3: None}[q])
    assert len(slots) == d
    return slots


def quantize_one(d, bits, Pi, books, x):
    """Encode one vector: (codes per slot [d] int, norm float32)."""
    x = np.asarray(x, np.float64)
    nu = float(np.sqrt(np.sum(x * x)))
    if nu == 0.0:
        return np.zeros(d, np.int64), np.float32(0.0)
    y = Pi @ (x / nu)
    angles, _ = polar_angles(y)
    codes = np.zeros(d, np.int64)
    for s, where in enumerate(_slot_order(d)):
        if where is None:
            continue
        level, i = where
        t = books[level - 1][1]
        codes[s] = int(np.sum(t < angles[level - 1][i]))
    return codes, np.float32(nu)


def dequant_one(d, bits, Pi, books, codes, nu):
    """Decode one record: x_hat = nu Pi^T y_hat, y_hat from the centroid angles."""
    L = levels(d)
    angles = [np.zeros(d >> level) for level in range(1, L + 1)]
    for s, where in enumerate(_slot_order(d)):
        if where is None:
            continue
        level, i = where
        angles[level - 1][i] = books[level - 1][0][codes[s]]
    y_hat = polar_reconstruct(angles, 1.0)
    return float(nu) * (Pi.T @ y_hat)


class PolarParams:
    """Data-oblivious state of one PolarQuant context (d, bits, seed)."""

    def __init__(self, d, bits, seed):
        if bits not in (1, 2, 3, 4):
            raise ValueError("bits in {1,2,3,4}")
        self.d, self.bits, self.seed = d, bits, seed
        self.L = levels(d)
        self.Pi = haar_rotation(d, seed)
        self.books = codebooks(d, bits)
        self.code_bytes, _ = record_sizes(d, bits, 0)


def quantize(p, X):
    """Records (codes [n, code_bytes] uint8, norms [n] float32) and the
    unpacked slot codes and exact angles (for the decision-band checks)."""
    X = np.asarray(X)
    n = X.shape[0]
    idx = np.zeros((n, p.d), np.int64)
    norms = np.zeros(n, np.float32)
    for v in range(n):
        idx[v], norms[v] = quantize_one(p.d, p.bits, p.Pi, p.books, X[v])
    return {"codes": pack_bits(idx, p.bits, p.code_bytes), "norms": norms, "idx": idx}


def dequant(p, codes, norms):
    """x_hat [n, d] from packed records."""
    idx = unpack_bits(codes, p.bits, p.d)
    return np.stack([dequant_one(p.d, p.bits, p.Pi, p.books, idx[v], norms[v])
                     for v in range(idx.shape[0])]) if idx.shape[0] else np.zeros((0, p.d))


def slot_margins(p, x):
    """Per record slot, the distance (unit-sphere scale) of the rotated point
    from the nearest decision boundary of that slot's angle: the radius of the
    pair times |sin(angle - threshold)|, minimised over thresholds (level 1
    also over the wrap at 0 = 2 pi); +inf for the spare slot or a zero vector."""
    x = np.asarray(x, np.float64)
    nu = float(np.sqrt(np.sum(x * x)))
    out = np.full(p.d, np.inf)
    if nu == 0.0:
        return out
    y = p.Pi @ (x / nu)
    angles, _ = polar_angles(y)
    radii = [np.hypot(y[0::2], y[1::2])]
    r = radii[0]
    while r.size > 1:
        r = np.hypot(r[0::2], r[1::2])
        radii.append(r)
    for s, where in enumerate(_slot_order(p.d)):
        if where is None:
            continue
        level, i = where
        t = p.books[level - 1][1]
        if level == 1:
            t = np.concatenate([[0.0], t])
        R = radii[level - 1][i]
        out[s] = R * np.min(np.abs(np.sin(angles[level - 1][i] - t)))
    return out
