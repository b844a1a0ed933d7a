"""Pins for the oracle's data-oblivious parameters (RNG, rotation, codebook).

Each test checks the oracle against something other than itself: published
test vectors and tables, closed forms, or brute force.
"""

import math
import os

import numpy as np
import pytest
from scipy import integrate, stats

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            rows.append([c.strip() for c in line.split("|")])
    return rows


def test_splitmix64_published_vector():
    # SplitMix64 started from state 0 (Steele, Lea, Flood 2014; the reference
    # C implementation by S. Vigna) returns 0xE220A8397B1DCDAF first.  Our
    # counter form reaches state 0 when seed = (stream + 1) * gamma.
    gamma = 0x9E3779B97F4A7C15
    out = O.splitmix64_stream(gamma, 0, 3)
    assert int(out[0]) == 0xE220A8397B1DCDAF
    assert int(out[1]) == 0x6E789E6AA1B965F4
    assert int(out[2]) == 0x06C45D188009454F


def test_gaussian_stream_is_standard_normal():
    g = O.gaussian_stream(123, 0, 200000)
    assert abs(g.mean()) < 4 / math.sqrt(len(g))
    assert abs(g.var() - 1.0) < 4 * math.sqrt(2.0 / len(g))
    assert stats.kstest(g, "norm").pvalue > 1e-3
    # streams are distinct
    assert not np.allclose(O.gaussian_stream(123, 1, 8), g[:8])


def test_haar_rotation_orthogonal_and_deterministic():
    for d in (8, 128, 200):
        P = O.haar_rotation(d, 7)
        assert np.abs(P.T @ P - np.eye(d)).max() < 1e-13
        assert np.array_equal(P, O.haar_rotation(d, 7))
    assert not np.allclose(O.haar_rotation(16, 1), O.haar_rotation(16, 2))


def test_haar_rotation_is_sign_normalised_qr_of_the_gaussian():
    # Pi must equal Q diag(sign R_ii) where G = Q R; equivalently Pi^T G is upper
    # triangular with a positive diagonal (uniqueness of that QR form).
    d = 24
    G = O.gaussian_stream(5, 0, d * d).reshape(d, d)
    R = O.haar_rotation(d, 5).T @ G
    assert np.abs(np.tril(R, -1)).max() < 1e-12
    assert (np.diag(R) > 0).all()


def test_rotated_coordinate_law():
    # suzuke blog, 第一步: a rotated coordinate tends to N(0, 1/d).  Exact law of
    # one coordinate of a Haar-rotated unit vector: y = 2B - 1 with
    # B ~ Beta((d-1)/2, (d-1)/2); var = 1/d, kurtosis = 3d/(d+2).
    d, n = 32, 3000
    u = np.zeros(d)
    u[0], u[1] = 0.96, 0.28       # a very uneven unit vector
    ys = np.array([(O.haar_rotation(d, s) @ u)[s % d] for s in range(n)])
    assert abs(ys.var() * d - 1.0) < 0.08
    kurt = np.mean(ys ** 4) / np.mean(ys ** 2) ** 2
    assert abs(kurt - 3 * d / (d + 2)) < 0.25
    a = (d - 1) / 2
    assert stats.kstest((ys + 1) / 2, stats.beta(a, a).cdf).pvalue > 1e-3
    assert stats.kstest(ys * math.sqrt(d), "norm").pvalue > 1e-4


def test_codebook_matches_max_1960_table():
    for N, outs, ends, dist in _read_table("max1960_gaussian.txt"):
        L = int(N)
        c, t = O.lloyd_max_gaussian(L)
        pos = c[L // 2:]
        assert np.allclose(pos, [float(v) for v in outs.split()], atol=6e-4), (L, pos)
        if ends != "-":
            assert np.allclose(t[L // 2:], [float(v) for v in ends.split()], atol=6e-4)
        assert abs(O.gaussian_distortion(c, t) - float(dist)) < 2e-5 + 1e-3 * float(dist)


def test_codebook_one_bit_closed_form():
    c, t = O.lloyd_max_gaussian(2)
    assert np.allclose(c, [-math.sqrt(2 / math.pi), math.sqrt(2 / math.pi)], atol=1e-15)
    assert t[0] == 0.0
    assert abs(O.gaussian_distortion(c, t) - (1 - 2 / math.pi)) < 1e-15


def test_codebook_optimality_conditions_and_distortion_integral():
    for L in (4, 8, 16):
        c, t = O.lloyd_max_gaussian(L)
        assert np.all(np.diff(c) > 0) and np.all(np.diff(t) > 0)
        assert np.allclose(c, -c[::-1], atol=0) and t[L // 2 - 1] == 0.0
        assert np.allclose(t, 0.5 * (c[1:] + c[:-1]), atol=1e-15)
        edges = [-np.inf] + list(t) + [np.inf]
        tot = 0.0
        for k in range(L):
            mass = stats.norm.cdf(edges[k + 1]) - stats.norm.cdf(edges[k])
            mean = integrate.quad(lambda x: x * stats.norm.pdf(x), edges[k], edges[k + 1])[0] / mass
            assert abs(mean - c[k]) < 1e-9
            tot += integrate.quad(lambda x: (x - c[k]) ** 2 * stats.norm.pdf(x), edges[k], edges[k + 1])[0]
        assert abs(tot - O.gaussian_distortion(c, t)) < 1e-9


def test_codebook_scaled_for_dimension():
    c1, t1 = O.lloyd_max_gaussian(8)
    c, t = O.codebook(200, 3)
    assert np.allclose(c, c1 / math.sqrt(200)) and np.allclose(t, t1 / math.sqrt(200))


def test_threshold_rule_equals_nearest_centroid():
    rng = np.random.default_rng(3)
    for w in (1, 2, 3, 4):
        c, t = O.codebook(128, w)
        y = rng.standard_normal(20000) / math.sqrt(128)
        idx = np.searchsorted(t, y, side="left")
        dist = np.abs(y[:, None] - c[None, :])
        nearest = np.argmin(dist, axis=1)   # first minimum = lower index on ties
        assert np.array_equal(idx, nearest)
        # a value exactly on threshold k takes the lower index k
        assert np.array_equal(np.searchsorted(t, t, side="left"), np.arange(len(t)))
        # the middle threshold is an exact tie between symmetric centroids
        mid = len(t) // 2
        assert np.argmin(np.abs(0.0 - c)) == mid == np.searchsorted(t, 0.0, side="left")


def test_make_params_modes_and_validation():
    p = O.make_params(128, 3, 0)
    assert (p.w, p.m, p.S.shape, len(p.c)) == (2, 128, (128, 128), 4)
    assert np.array_equal(p.S, O.jl_matrix(128, 128, 0))
    assert abs(p.alpha - math.sqrt(math.pi / 2) / 128) < 1e-18
    q = O.make_params(64, 4, 1, "mse")
    assert (q.w, q.m, len(q.c)) == (4, 0, 16)
    for bad in [(7, 3, "prod"), (0, 3, "prod"), (128, 1, "prod"), (128, 5, "prod"), (128, 5, "mse")]:
        with pytest.raises(ValueError):
            O.make_params(bad[0], bad[1], 0, bad[2])
