"""Pins for the oracle's quantizer, estimator and dequantizer.

Besides closed forms and identities, the statistical pins reproduce the
figures the pages print (tests/golden/pages_figures.txt): MSE ~0.03 at 3
bits, within ~2.7x of the 4^-b lower bound and ~1.45x at 1 bit, an unbiased
two-stage estimator, and the 2/pi bias of the MSE-only 1-bit quantizer.  The
``planted`` tests swap a deliberate mistake into the oracle and check that a
pin catches it.
"""

import math
import os
from dataclasses import replace

import numpy as np
import pytest
from scipy.special import gammaln

import oracle as O
from oracle import quant as OQ

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _figures():
    out = {}
    with open(os.path.join(GOLDEN, "pages_figures.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v, _ = [c.strip() for c in line.split("|")]
                out[k] = float(v)
    return out


FIG = _figures()


def _unit(n, d, seed):
    U = np.random.default_rng(seed).standard_normal((n, d))
    return U / np.linalg.norm(U, axis=1, keepdims=True)


# ------------------------------------------------------------ layout / packing
def test_pack_bits_hand_example():
    # codes 1,2,3,0,3 at 2 bits -> bit stream (LSB first) 10 01 11 00 11
    # byte0 = b0..b7 = 1,0,0,1,1,1,0,0 -> 0b00111001 = 0x39 ; byte1 = 1,1 -> 0x03
    packed = O.pack_bits(np.array([[1, 2, 3, 0, 3]]), 2, 16)
    assert packed.shape == (1, 16)
    assert packed[0, 0] == 0x39 and packed[0, 1] == 0x03 and not packed[0, 2:].any()
    # 3-bit codes straddle bytes: 5,6 -> 101 011 -> bits 1,0,1,0,1,1 -> 0x35
    assert O.pack_bits(np.array([[5, 6]]), 3, 16)[0, 0] == 0x35


def test_pack_unpack_roundtrip():
    rng = np.random.default_rng(0)
    for w, d in [(1, 200), (2, 128), (3, 200), (4, 64)]:
        v = rng.integers(0, 2 ** w, (50, d))
        cb, _ = O.record_sizes(d, w, 0)
        assert np.array_equal(O.unpack_bits(O.pack_bits(v, w, cb), w, d), v)


def test_pack_planes_hand_example():
    # d = 16 at 3 bits: codes 5 (101), 2 (010), 7 (111), 0 at coordinates 0..3
    # and 6 (110) at coordinate 15.  Plane p holds bit p of code i at bit i:
    # plane 0 = 1,0,1,0,...,0 -> bytes 0x05 0x00; plane 1 = 0,1,1,0,...,1 ->
    # 0x06 0x80; plane 2 = 1,0,1,0,...,1 -> 0x05 0x80
    v = np.zeros((1, 16), np.int64)
    v[0, :4] = [5, 2, 7, 0]
    v[0, 15] = 6
    packed = O.pack_planes(v, 3, 16, 16)
    assert packed[0].tolist() == [0x05, 0x00, 0x06, 0x80, 0x05, 0x80] + [0] * 10
    assert np.array_equal(O.unpack_planes(packed, 3, 16), v)


def test_planes_are_the_stream_transposed():
    # bit p of code i: stream bit i w + p, plane bit p d + i
    rng = np.random.default_rng(1)
    for w, d in [(1, 24), (2, 64), (3, 128), (4, 40)]:
        v = rng.integers(0, 2 ** w, (20, d))
        cb, _ = O.record_sizes(d, w, 0)
        st = np.unpackbits(O.pack_bits(v, w, cb), axis=1, bitorder="little")
        pl = np.unpackbits(O.pack_planes(v, w, d, cb), axis=1, bitorder="little")
        assert pl.shape == st.shape
        for p in range(w):
            assert np.array_equal(pl[:, p * d:(p + 1) * d], st[:, p:w * d:w])
        assert not pl[:, w * d:].any()
        assert np.array_equal(O.unpack_planes(O.pack_planes(v, w, d, cb), w, d), v)


def test_records_by_mode():
    # prod records (keys) keep the bit stream, MSE-only records (values) the planes
    X = np.random.default_rng(2).standard_normal((30, 64))
    for mode, packer in (("prod", lambda p, i: O.pack_bits(i, p.w, O.record_sizes(p.d, p.w, p.m)[0])),
                         ("mse", lambda p, i: O.pack_planes(i, p.w, p.d, O.record_sizes(p.d, p.w, p.m)[0]))):
        p = O.make_params(64, 3, 5, mode)
        r = O.quantize(p, X, return_unpacked=True)
        assert np.array_equal(r["codes"], packer(p, r["idx"]))
        assert np.array_equal(O.unpack_codes(p, r["codes"]), r["idx"])
        xh = O.dequant(p, r["codes"], r["signs"], r["norms"], r["rnorms"])
        assert np.allclose(xh[:, :], (p.c[r["idx"]] @ p.Pi) * r["norms"][:, None].astype(np.float64)
                           + (0 if mode == "mse" else xh - (p.c[r["idx"]] @ p.Pi) * r["norms"][:, None]))


def test_record_sizes():
    assert O.record_sizes(128, 2, 128) == (32, 16)
    assert O.record_sizes(128, 1, 128) == (16, 16)
    assert O.record_sizes(128, 3, 128) == (48, 16)
    assert O.record_sizes(200, 1, 200) == (32, 32)
    assert O.record_sizes(200, 3, 200) == (80, 32)
    assert O.record_sizes(128, 3, 0) == (48, 0)


# --------------------------------------------------- scalar vs batched, cases
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_batched_equals_scalar(bits):
    p = O.make_params(128, bits, 0)
    rng = np.random.default_rng(1)
    X = rng.standard_normal((64, 128)).astype(np.float32)
    Q = rng.standard_normal((3, 128))
    r = O.quantize(p, X, chunk=17, return_unpacked=True)
    L = O.scores(p, Q, r["codes"], r["signs"], r["norms"], r["rnorms"])
    for i in range(len(X)):
        idx, sb, nu, g = O.quantize_one(p, X[i])
        assert np.array_equal(idx, r["idx"][i]) and np.array_equal(sb, r["sbits"][i])
        assert nu == r["norms"][i] and g == r["rnorms"][i]
        for j in range(len(Q)):
            l1 = O.scores_one(p, Q[j], r["codes"][i], r["signs"][i], r["norms"][i], r["rnorms"][i])
            assert abs(l1 - L[j, i]) <= 1e-12 * max(1.0, abs(l1))


def test_zero_vector_encoding():
    p = O.make_params(64, 3, 0)
    X = np.zeros((3, 64), np.float32)
    X[1, 5] = 2.0
    r = O.quantize(p, X)
    for i in (0, 2):
        assert not r["codes"][i].any() and not r["signs"][i].any()
        assert r["norms"][i] == 0 and r["rnorms"][i] == 0
    assert r["norms"][1] == 2.0
    L = O.scores(p, np.ones((1, 64)), r["codes"], r["signs"], r["norms"], r["rnorms"])
    assert L[0, 0] == 0.0 and L[0, 2] == 0.0


def test_norm_is_rounded_float64_length():
    p = O.make_params(32, 2, 0)
    X = np.random.default_rng(2).standard_normal((100, 32)).astype(np.float32)
    r = O.quantize(p, X)
    exact = np.sqrt((X.astype(np.float64) ** 2).sum(1))
    assert np.array_equal(r["norms"], exact.astype(np.float32))


def test_scale_invariance_of_codes():
    p = O.make_params(64, 4, 3)
    X = np.random.default_rng(4).standard_normal((50, 64))
    a, b = O.quantize(p, X), O.quantize(p, 4.0 * X)
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["signs"], b["signs"])
    assert np.allclose(4.0 * a["norms"], b["norms"])


# ------------------------------------------------------------ identities
def test_sketch_identity_and_residual_norm():
    # JL of the stage-1 error in x's coordinates equals S Pi^T applied to the
    # rotated residual; its length equals gamma (Pi orthogonal).
    p = O.make_params(96, 3, 5)
    X = np.random.default_rng(6).standard_normal((40, 96))
    r = O.quantize(p, X, return_unpacked=True)
    resid = r["y"] - p.c[r["idx"]]
    z_rot = resid @ (p.S @ p.Pi.T).T
    assert np.abs(z_rot - r["z"]).max() < 1e-12
    assert np.allclose(np.linalg.norm(resid, axis=1), r["rnorms"], rtol=1e-6)
    assert np.array_equal((r["z"] >= 0).astype(int), r["sbits"])


@pytest.mark.parametrize("mode,bits", [("prod", 2), ("prod", 3), ("prod", 4), ("mse", 3), ("mse", 1)])
def test_scores_equal_query_dot_dequant(mode, bits):
    p = O.make_params(64, bits, 9, mode)
    rng = np.random.default_rng(10)
    r = O.quantize(p, rng.standard_normal((30, 64)))
    Q = rng.standard_normal((5, 64))
    L = O.scores(p, Q, r["codes"], r["signs"], r["norms"], r["rnorms"])
    Xh = O.dequant(p, r["codes"], r["signs"], r["norms"], r["rnorms"])
    assert np.abs(L - Q @ Xh.T).max() < 1e-12 * max(1.0, np.abs(L).max())


def test_dequant_mse_is_rotated_back_centroids():
    p = O.make_params(32, 2, 1, "mse")
    r = O.quantize(p, np.eye(32)[:4] * 3.0, return_unpacked=True)
    Xh = O.dequant(p, r["codes"], None, r["norms"], None)
    for i in range(4):
        assert np.allclose(Xh[i], 3.0 * p.Pi.T @ p.c[r["idx"][i]])


# ------------------------------------------------------ figures from the pages
def _mse_unit(bits, d=128, n=20000, seed=0):
    p = O.make_params(d, bits, seed, "mse")
    U = _unit(n, d, 100 + bits)
    r = O.quantize(p, U)
    Xh = O.dequant(p, r["codes"], None, r["norms"], None)
    return float(np.mean(np.sum((U - Xh) ** 2, axis=1)))


def test_mse_3bit_near_pages_figure():
    # suzuke blog, 第三步: 3 bits -> MSE 0.03 (a 1-significant-figure value).
    mse = _mse_unit(3)
    assert abs(mse - FIG["mse_unit_3bit"]) < 0.005
    # and it matches the codebook's Gaussian design distortion within 3%
    c, t = O.lloyd_max_gaussian(8)
    assert abs(mse / O.gaussian_distortion(c, t) - 1) < 0.03


def test_mse_ratio_to_lower_bound():
    # xujun.org note 189244, 性能数据: within ~2.7x of the 4^-b bound at every
    # width, ~1.45x at 1 bit.
    ratios = [_mse_unit(b, n=8000) * 4 ** b for b in (1, 2, 3, 4)]
    assert all(r <= FIG["ratio_to_bound_max"] for r in ratios), ratios
    assert abs(ratios[0] - FIG["ratio_to_bound_1bit"]) < 0.03, ratios
    assert ratios == sorted(ratios)          # rises towards sqrt(3) pi / 2


def _estimator_errors(bits, d, seeds, q, x, mode="prod"):
    out = []
    for s in seeds:
        p = O.make_params(d, bits, s, mode)
        r = O.quantize(p, x[None, :])
        out.append(O.scores(p, q[None, :], r["codes"], r["signs"], r["norms"], r["rnorms"])[0, 0])
    return np.array(out)


def _fixed_pair(d):
    rng = np.random.default_rng(77)
    x = rng.standard_normal(d) * 2.0
    q = 0.6 * x / np.linalg.norm(x) * 3.0 + rng.standard_normal(d)
    return q, x


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_estimator_unbiased_over_seeds(bits):
    # xujun.org note 189244, 第二步：QJL: the expected inner product is unchanged.
    d = 64
    q, x = _fixed_pair(d)
    est = _estimator_errors(bits, d, range(2500), q, x)
    err = est - q @ x
    z = err.mean() / (err.std(ddof=1) / math.sqrt(len(err)))
    assert abs(z) < 4.0, (err.mean(), z)


def test_mse_only_one_bit_has_two_over_pi_bias():
    # xujun.org note 189244, 第二步：QJL: the MSE-optimal 1-bit quantizer is
    # biased by 2/pi in high dimension.  Exact factor for Haar Pi:
    # sqrt(2d/pi) Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)).
    d = 128
    kappa = math.sqrt(2 * d / math.pi) * math.exp(gammaln(d / 2) - gammaln((d + 1) / 2)) / math.sqrt(math.pi)
    assert abs(kappa - 0.637864) < 1e-6
    assert abs(kappa - FIG["bias_mse_1bit"]) < 0.002
    x = np.random.default_rng(1).standard_normal(d)
    est = _estimator_errors(1, d, range(600), x, x, mode="mse")
    ratio = est / (x @ x)
    se = ratio.std(ddof=1) / math.sqrt(len(ratio))
    assert abs(ratio.mean() - kappa) < 4 * se + 1e-4, (ratio.mean(), kappa, se)
    # the two-stage estimator at the same total budget has no such bias
    est2 = _estimator_errors(2, d, range(600), x, x)
    r2 = est2 / (x @ x)
    assert abs(r2.mean() - 1.0) < 4 * r2.std(ddof=1) / math.sqrt(len(r2))


def _variance_case(alpha_override=None):
    d, n = 48, 3000
    base = O.make_params(d, 3, 0)
    rng = np.random.default_rng(8)
    x = rng.standard_normal(d)
    q = rng.standard_normal(d)
    vals = []
    for s in range(n):
        p = replace(base, S=O.jl_matrix(d, d, 1000 + s))
        if alpha_override is not None:
            p = _AlphaParams(p, alpha_override)
        r = O.quantize(p, x[None, :], return_unpacked=True)
        vals.append(O.scores(p, q[None, :], r["codes"], r["signs"], r["norms"], r["rnorms"])[0, 0])
    r = O.quantize(base, x[None, :], return_unpacked=True)
    nu = np.linalg.norm(x)
    resid = r["y"][0] - base.c[r["idx"][0]]
    gamma = np.linalg.norm(resid)
    q_rot = base.Pi @ q
    var = nu ** 2 * ((math.pi / 2) * gamma ** 2 * (q @ q) - (resid @ q_rot) ** 2) / d
    mean = nu * (q_rot @ r["y"][0])                    # = <q, x>
    return np.array(vals), var, mean


class _AlphaParams:
    """TQParams proxy with a different residual scale (planted mistakes)."""

    def __init__(self, p, alpha):
        self._p, self._alpha = p, alpha

    def __getattr__(self, k):
        return getattr(self._p, k)

    @property
    def alpha(self):
        return self._alpha


def test_estimator_variance_closed_form():
    # Given Pi, over S: Var = nu^2 ((pi/2) gamma^2 |q|^2 - <r, Pi q>^2) / m.
    vals, var, mean = _variance_case()
    n = len(vals)
    assert abs(vals.var(ddof=1) / var - 1) < 0.1
    assert abs(vals.mean() - mean) < 4 * math.sqrt(var / n)


# ------------------------------------------------------------ planted mistakes
def test_planted_wrong_alpha_is_caught():
    d = 48
    wrong = math.sqrt(2 / math.pi) / d           # inverted constant
    vals, var, mean = _variance_case(alpha_override=wrong)
    se = vals.std(ddof=1) / math.sqrt(len(vals))
    assert abs(vals.mean() - mean) > 4 * se or abs(vals.var(ddof=1) / var - 1) > 0.1


def test_planted_dropped_residual_term_is_caught(monkeypatch):
    d = 64
    q, x = _fixed_pair(d)
    good = _estimator_errors(3, d, range(800), q, x) - q @ x
    monkeypatch.setattr(O.TQParams, "alpha", property(lambda self: 0.0))
    bad = _estimator_errors(3, d, range(800), q, x) - q @ x
    z_good = good.mean() / (good.std(ddof=1) / math.sqrt(len(good)))
    z_bad = bad.mean() / (bad.std(ddof=1) / math.sqrt(len(bad)))
    assert abs(z_good) < 4 and abs(z_bad) > 4


def test_planted_transposed_rotation_is_caught(monkeypatch):
    # Using Pi instead of Pi^T to return from rotated coordinates breaks the
    # dequant/scores identity.
    p = O.make_params(32, 3, 2)
    rng = np.random.default_rng(3)
    r = O.quantize(p, rng.standard_normal((10, 32)))
    Q = rng.standard_normal((2, 32))
    L = O.scores(p, Q, r["codes"], r["signs"], r["norms"], r["rnorms"])
    bad = replace(p, Pi=p.Pi.T.copy())
    Xh = O.dequant(bad, r["codes"], r["signs"], r["norms"], r["rnorms"])
    assert np.abs(L - Q @ Xh.T).max() > 1e-3


def test_planted_wrong_tie_rule_is_caught():
    # A "<=" threshold comparison moves exact ties to the upper index, which the
    # nearest-centroid brute force (lower index on ties) rejects.
    c, t = O.codebook(128, 2)
    y = np.array([0.0, 0.3, -0.01, 0.05])   # 0.0 is the middle threshold
    right = np.searchsorted(t, y, side="left")
    wrong = np.searchsorted(t, y, side="right")
    nearest = np.argmin(np.abs(y[:, None] - c[None, :]), axis=1)
    assert np.array_equal(right, nearest) and not np.array_equal(wrong, nearest)


def test_stage2_from_codes_reproduces_quantize():
    p = O.make_params(64, 3, 4)
    X = np.random.default_rng(12).standard_normal((20, 64))
    r = O.quantize(p, X, return_unpacked=True)
    for i in range(20):
        g, z, sb = O.stage2_from_codes(p, X[i], r["idx"][i])
        assert abs(g - r["rnorms"][i]) < 1e-6 * max(g, 1e-3)
        assert np.abs(z - r["z"][i]).max() < 1e-12 and np.array_equal(sb, r["sbits"][i])
    # a different (neighbouring) code choice changes the residual by the centroid gap
    alt = r["idx"][0].copy()
    alt[0] = alt[0] + 1 if alt[0] < 3 else alt[0] - 1
    g2, _, _ = O.stage2_from_codes(p, X[0], alt)
    y0 = (p.Pi @ (X[0] / np.linalg.norm(X[0])))[0]
    want = np.sqrt(r["rnorms"][0] ** 2 - (y0 - p.c[r["idx"][0][0]]) ** 2 + (y0 - p.c[alt[0]]) ** 2)
    assert abs(g2 - want) < 1e-6
