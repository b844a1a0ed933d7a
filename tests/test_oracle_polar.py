"""Pins of the PolarQuant oracle (oracle/polar.py) against what the pages and
the mathematics fix, independently of the oracle's own arithmetic:

* the recursive polar transform is invertible (exact angles reconstruct y);
* the angle laws: level 1 uniform on [0, 2 pi); level l >= 2 with sin^2(phi)
  ~ Beta(k/2, k/2), k = 2^(l-1) -- checked by a KS test on random sphere
  points against SciPy's regularized incomplete beta (not used by the oracle);
* every level's codebook satisfies the Lloyd-Max conditions under SciPy's
  adaptive quadrature, and the 1-bit level-2 codebook has the closed form
  centroids 1/2 and pi/2 - 1/2 (f_2 = sin 2 phi);
* the reconstruction MSE of unit vectors equals the closed form
  2 - 2 E<y, y_hat>, E<y, y_hat> = sinc(pi / 2^b) prod_l 2 E[cos phi cos phi_hat]
  (angles at different levels are independent), within Monte-Carlo error;
* the record layout, on hand-computed vectors.
"""

import math

import numpy as np
import pytest

import oracle.polar as P
from oracle import codebook as scalar_codebook
from oracle.params import gaussian_distortion, lloyd_max_gaussian

scipy = pytest.importorskip("scipy")
from scipy import integrate, special, stats  # noqa: E402


@pytest.mark.parametrize("d", [8, 16, 64, 256])
def test_polar_transform_round_trip(d):
    rng = np.random.default_rng(d)
    for _ in range(20):
        y = rng.standard_normal(d)
        angles, r = P.polar_angles(y)
        assert len(angles) == P.levels(d)
        assert [a.size for a in angles] == [d >> level for level in range(1, P.levels(d) + 1)]
        assert abs(r - np.linalg.norm(y)) < 1e-12 * r
        assert np.abs(P.polar_reconstruct(angles, r) - y).max() < 1e-12 * r
        assert (angles[0] >= 0).all() and (angles[0] < 2 * math.pi).all()
        assert all(((a >= 0) & (a <= math.pi / 2)).all() for a in angles[1:])


def test_angle_laws_ks():
    d, n = 64, 20000
    rng = np.random.default_rng(5)
    Y = rng.standard_normal((n, d))
    Y /= np.linalg.norm(Y, axis=1, keepdims=True)
    per_level = [[] for _ in range(P.levels(d))]
    for y in Y[:4000]:
        angles, _ = P.polar_angles(y)
        for level, a in enumerate(angles):
            per_level[level].append(a)
    for level in range(1, P.levels(d) + 1):
        a = np.concatenate(per_level[level - 1])
        if level == 1:
            cdf = lambda x: x / (2 * math.pi)                       # noqa: E731
        else:
            k = 2 ** (level - 1)
            cdf = lambda x, k=k: special.betainc(k / 2, k / 2, np.sin(x) ** 2)  # noqa: E731
        res = stats.kstest(a, cdf)
        assert res.pvalue > 1e-3, (level, res)
    # a planted mistake is caught: the level-3 angles are not level-2 distributed
    a3 = np.concatenate(per_level[2])
    assert stats.kstest(a3, lambda x: special.betainc(1.0, 1.0, np.sin(x) ** 2)).pvalue < 1e-6


@pytest.mark.parametrize("level", [2, 3, 5, 8])
def test_angle_density_is_the_beta_law(level):
    k = 2 ** (level - 1)
    tot = integrate.quad(lambda x: float(P.angle_density(level, x)), 0, math.pi / 2)[0]
    assert abs(tot - 1.0) < 1e-10
    for phi in (0.1, 0.5, math.pi / 4, 1.2):
        u = math.sin(phi) ** 2
        beta_pdf = stats.beta(k / 2, k / 2).pdf(u) * 2 * math.sin(phi) * math.cos(phi)
        assert abs(float(P.angle_density(level, phi)) - beta_pdf) < 1e-9 * max(1.0, beta_pdf)


@pytest.mark.parametrize("d,bits", [(64, 1), (64, 3), (128, 2), (256, 4)])
def test_codebooks_lloyd_max_conditions(d, bits):
    books = P.codebooks(d, bits)
    n = 2 ** bits
    c1, t1 = books[0]
    assert np.allclose(c1, (np.arange(n) + 0.5) * 2 * math.pi / n)
    assert np.allclose(t1, np.arange(1, n) * 2 * math.pi / n)
    for level in range(2, P.levels(d) + 1):
        c, t = books[level - 1]
        assert c.size == n and t.size == n - 1
        assert np.all(np.diff(c) > 0) and np.allclose(c + c[::-1], math.pi / 2)
        assert np.allclose(t, 0.5 * (c[:-1] + c[1:]), atol=1e-14)
        edges = [0.0] + list(t) + [math.pi / 2]
        f = lambda x: float(P.angle_density(level, x))           # noqa: E731
        for i in range(n):
            m0 = integrate.quad(f, edges[i], edges[i + 1], epsabs=1e-14, epsrel=1e-12)[0]
            m1 = integrate.quad(lambda x: x * f(x), edges[i], edges[i + 1], epsabs=1e-14, epsrel=1e-12)[0]
            assert abs(m1 / m0 - c[i]) < 1e-9, (level, i, m1 / m0, c[i])


def test_level2_one_bit_closed_form():
    # f_2(phi) = sin(2 phi); cells [0, pi/4], [pi/4, pi/2]; mean of the first
    # cell = (1/4) / (1/2) = 1/2
    c, t = P.lloyd_max_angle(2, 2)
    assert abs(t[0] - math.pi / 4) < 1e-15
    assert abs(c[0] - 0.5) < 1e-12 and abs(c[1] - (math.pi / 2 - 0.5)) < 1e-12


def _closed_form_mse(d, bits):
    books = P.codebooks(d, bits)
    n = 2 ** bits
    w = 2 * math.pi / n
    prod = math.sin(w / 2) / (w / 2)                     # E cos(theta - theta_hat)
    for level in range(2, P.levels(d) + 1):
        c, t = books[level - 1]
        edges = [0.0] + list(t) + [math.pi / 2]
        ecc = sum(math.cos(c[i]) * integrate.quad(lambda x: math.cos(x) * float(P.angle_density(level, x)),
                                                  edges[i], edges[i + 1])[0] for i in range(n))
        prod *= 2.0 * ecc                                # E[cos cos_hat] + E[sin sin_hat]
    return 2.0 - 2.0 * prod


@pytest.mark.parametrize("bits", [1, 3])
def test_mse_closed_form_vs_monte_carlo(bits):
    d, nvec = 64, 2000
    p = P.PolarParams(d, bits, seed=3)
    rng = np.random.default_rng(11)
    X = rng.standard_normal((nvec, d))
    rec = P.quantize(p, X)
    Xh = P.dequant(p, rec["codes"], rec["norms"])
    U = X / np.linalg.norm(X, axis=1, keepdims=True)
    Uh = Xh / rec["norms"].astype(np.float64)[:, None]
    err = np.sum((U - Uh) ** 2, axis=1)
    assert np.allclose(np.linalg.norm(Uh, axis=1), 1.0, atol=1e-6)   # |y_hat| = 1
    want = _closed_form_mse(d, bits)
    se = err.std() / math.sqrt(nvec)
    assert abs(err.mean() - want) < 4 * se + 2e-6, (err.mean(), want, se)


def test_mse_against_scalar_codes():
    # The pages' reading of PolarQuant, every angle at b bits, against the
    # per-coordinate Lloyd-Max codes of the MSE-only stage at the same b bits
    # (Gaussian design distortion D_b per coordinate; d coordinates of
    # variance 1/d): the scalar codes reach the lower MSE at every b here, and
    # PolarQuant stays within 4x of the 4^-b lower bound.
    d = 128
    for bits in (1, 2, 3, 4):
        polar = _closed_form_mse(d, bits)
        c, t = lloyd_max_gaussian(2 ** bits)
        scalar = gaussian_distortion(c, t)
        assert scalar < polar < 4.0 * 4.0 ** -bits, (bits, scalar, polar)
    assert scalar_codebook(d, 3)[0].size == 8


def test_record_layout_hand_computed():
    d, bits = 16, 3
    p = P.PolarParams(d, bits, seed=0)
    p.Pi = np.eye(d)                                     # identity rotation: angles of x itself
    n = 2 ** bits
    # x = e_4 (first coordinate of quarter 1): every angle is 0 except the
    # level-3 angle of quarters 0/1, atan2(R1 = 1, R0 = 0) = pi/2, which is
    # above every threshold (code n - 1) and sits in the spare slot of
    # quarter 1 = slot 2 (d/4) - 1 = 7
    x = np.zeros(d)
    x[4] = 1.0
    codes, nu = P.quantize_one(d, bits, p.Pi, p.books, x)
    want = np.zeros(d, np.int64)
    want[7] = n - 1
    assert np.array_equal(codes, want) and nu == 1.0
    rec = P.quantize(p, x[None])
    # slot 7 holds bits 21..23 of the bit stream: byte 2 bits 5..7
    expect = np.zeros(p.code_bytes, np.uint8)
    expect[2] = 0b11100000
    assert np.array_equal(rec["codes"][0], expect)
    # x = e_1: level-1 angle of pair 0 is pi/2 -> code #{k: 2 pi k / 8 < pi/2} = 1
    # (the tie at pi/2 takes the lower index); level-2 angle 0, ...
    x = np.zeros(d)
    x[1] = 1.0
    codes, _ = P.quantize_one(d, bits, p.Pi, p.books, x)
    want = np.zeros(d, np.int64)
    want[0] = 1
    assert np.array_equal(codes, want)
    # decoding the first record gives the centroid direction
    y = P.dequant(p, rec["codes"], rec["norms"])[0]
    assert abs(np.linalg.norm(y) - 1.0) < 1e-12


def test_zero_vector_and_scale_invariance():
    p = P.PolarParams(32, 2, seed=1)
    rec = P.quantize(p, np.zeros((1, 32)))
    assert not rec["codes"].any() and rec["norms"][0] == 0
    assert not P.dequant(p, rec["codes"], rec["norms"]).any()
    x = np.random.default_rng(2).standard_normal((3, 32))
    a, b = P.quantize(p, x), P.quantize(p, 1000.0 * x)
    assert np.array_equal(a["codes"], b["codes"])
