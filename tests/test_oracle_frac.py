"""Pins of the fractional-width oracle (oracle/frac.py), independent of its own
arithmetic:

* with equal widths in both halves the scheme is the integer-width method:
  codes, signs, norms, logits and reconstructions equal the (separately
  pinned) integer oracle's;
* with unequal widths each half takes exactly the codes of the integer
  context at its own width (same seed, so the same Pi), and the centroids of
  that width;
* the record layout on a hand-computed vector (identity rotation);
* the stage-1 MSE of unit vectors is the mean of the two widths' Gaussian
  design distortions (within 3%), strictly between the neighbouring integer
  widths' measured MSE;
* the estimator is unbiased over seeds, and its variance over the JL matrix
  follows the closed form nu^2 ((pi/2) gamma^2 |q|^2 - <r, Pi q>^2) / m and
  lies strictly between the integer widths' on the same pair;
* planted mistakes (swapped halves, floor/ceil swapped, planes reversed) fail.
"""

import math

import numpy as np
import pytest

import oracle as O
import oracle.frac as F


def _unit(n, d, seed):
    x = np.random.default_rng(seed).standard_normal((n, d))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


def test_widths_of_the_two_settings():
    p = F.FracParams(128, 5, 0)
    assert (p.w_hi, p.w_lo) == (2, 1) and p.code_bytes == 24 and p.sign_bytes == 16
    p = F.FracParams(128, 7, 0)
    assert (p.w_hi, p.w_lo) == (3, 2) and p.code_bytes == 40
    # average bits per coordinate: codes + one sign bit per JL row (m = d)
    for hb in (5, 7):
        p = F.FracParams(256, hb, 1)
        assert (8 * p.code_bytes + p.m) / p.d == hb / 2


@pytest.mark.parametrize("d,w", [(64, 1), (128, 2), (96, 3)])
def test_equal_widths_reduce_to_the_integer_method(d, w):
    pf = F.FracParams(d, None, 3, widths=(w, w))
    pi = O.make_params(d, w + 1, 3)
    X = np.random.default_rng(d).standard_normal((300, d)) * 2.0
    X[7] = 0.0
    rf = F.quantize(pf, X, return_unpacked=True)
    ri = O.quantize(pi, X, return_unpacked=True)
    assert np.array_equal(rf["idx"], ri["idx"]) and np.array_equal(rf["sbits"], ri["sbits"])
    assert np.array_equal(rf["signs"], ri["signs"][:, :pf.sign_bytes])
    assert np.array_equal(rf["norms"], ri["norms"]) and np.array_equal(rf["rnorms"], ri["rnorms"])
    assert np.array_equal(F.unpack(pf, rf["codes"]), ri["idx"])
    Q = np.random.default_rng(5).standard_normal((4, d))
    sf = F.scores(pf, Q, rf["codes"], rf["signs"], rf["norms"], rf["rnorms"])
    si = O.scores(pi, Q, ri["codes"], ri["signs"], ri["norms"], ri["rnorms"])
    assert np.abs(sf - si).max() < 1e-12 * np.abs(si).max()
    df = F.dequant(pf, rf["codes"], rf["signs"], rf["norms"], rf["rnorms"])
    di = O.dequant(pi, ri["codes"], ri["signs"], ri["norms"], ri["rnorms"])
    assert np.abs(df - di).max() < 1e-12 * np.abs(di).max()


@pytest.mark.parametrize("hb", [5, 7])
def test_each_half_is_coded_at_its_own_width(hb):
    d = 128
    p = F.FracParams(d, hb, 4)
    hi, lo = O.make_params(d, p.w_hi + 1, 4), O.make_params(d, p.w_lo + 1, 4)
    X = np.random.default_rng(9).standard_normal((200, d))
    r = F.quantize(p, X, return_unpacked=True)
    h = d // 2
    assert np.array_equal(r["idx"][:, :h], O.quantize(hi, X, return_unpacked=True)["idx"][:, :h])
    assert np.array_equal(r["idx"][:, h:], O.quantize(lo, X, return_unpacked=True)["idx"][:, h:])
    chat = p.centroids(r["idx"])
    assert np.array_equal(chat[:, :h], hi.c[r["idx"][:, :h]]) and np.array_equal(chat[:, h:], lo.c[r["idx"][:, h:]])
    # the residual and the sketch are those of the mixed centroids
    assert np.allclose(r["rnorms"], np.linalg.norm(r["y"] - chat, axis=1), rtol=1e-6)


def test_record_layout_hand_computed():
    d = 32
    p = F.FracParams(d, 5, 0)                 # w_hi = 2 (4 levels), w_lo = 1
    p.Pi = np.eye(d)
    x = np.zeros((1, d))
    x[0, 0] = 3.0
    r = F.quantize(p, x, return_unpacked=True)
    # y = e_0: coordinate 0 above every threshold -> code 3; the other y_i = 0
    # lie on the middle threshold (0) and take the lower index: 1 in the
    # 4-level half (one threshold below 0), 0 in the 2-level half
    want = np.array([3] + [1] * 15 + [0] * 16)
    assert np.array_equal(r["idx"][0], want)
    # quarter 0 (coords 0-7): plane 0 = 0xff, plane 1 = 0x01; quarter 1:
    # plane 0 = 0xff, plane 1 = 0x00; quarters 2, 3: one plane each, zero
    assert r["codes"][0].tolist() == [0xFF, 0x01, 0xFF, 0x00, 0x00, 0x00]
    assert r["norms"][0] == 3.0


def test_zero_vector_and_round_trip():
    p = F.FracParams(64, 7, 2)
    r = F.quantize(p, np.zeros((2, 64)))
    assert not r["codes"].any() and not r["signs"].any() and not r["norms"].any() and not r["rnorms"].any()
    idx = np.concatenate([np.random.default_rng(1).integers(0, 8, (5, 32)),
                          np.random.default_rng(2).integers(0, 4, (5, 32))], axis=1)
    assert np.array_equal(F.unpack(p, F.pack(p, idx)), idx)


def _mse_stage1(p, U):
    r = F.quantize(p, U, return_unpacked=True) if isinstance(p, F.FracParams) else O.quantize(p, U, return_unpacked=True)
    chat = p.centroids(r["idx"]) if isinstance(p, F.FracParams) else p.c[r["idx"]]
    return float(np.mean(np.sum((r["y"] - chat) ** 2, axis=1)))


@pytest.mark.parametrize("hb", [5, 7])
def test_mse_between_neighbouring_widths(hb):
    d = 128
    U = _unit(6000, d, 31)
    p = F.FracParams(d, hb, 0)
    mse = _mse_stage1(p, U)
    D = [O.gaussian_distortion(*O.lloyd_max_gaussian(2 ** w)) for w in (p.w_hi, p.w_lo)]
    assert abs(mse / (0.5 * (D[0] + D[1])) - 1) < 0.03, (mse, D)
    lo_int = _mse_stage1(O.make_params(d, p.w_hi + 1, 0), U)     # more bits: lower MSE
    hi_int = _mse_stage1(O.make_params(d, p.w_lo + 1, 0), U)
    assert lo_int < mse < hi_int, (lo_int, mse, hi_int)


def _pair(d):
    rng = np.random.default_rng(77)
    x = rng.standard_normal(d) * 2.0
    q = 0.6 * x / np.linalg.norm(x) * 3.0 + rng.standard_normal(d)
    return q, x


@pytest.mark.parametrize("hb", [5, 7])
def test_estimator_unbiased_over_seeds(hb):
    d = 64
    q, x = _pair(d)
    err = []
    for s in range(1500):
        p = F.FracParams(d, hb, s)
        r = F.quantize(p, x[None, :])
        err.append(F.scores(p, q[None, :], r["codes"], r["signs"], r["norms"], r["rnorms"])[0, 0] - q @ x)
    err = np.array(err)
    z = err.mean() / (err.std(ddof=1) / math.sqrt(len(err)))
    assert abs(z) < 4.0, (err.mean(), z)


def _variance_over_S(make, d=64, n=2500):
    """Estimates over JL matrices for a fixed Pi and pair, and the closed form."""
    base = make(0)
    rng = np.random.default_rng(8)
    x, q = rng.standard_normal(d), rng.standard_normal(d)
    vals = []
    for s in range(n):
        base.S = O.jl_matrix(d, d, 1000 + s)
        if isinstance(base, F.FracParams):
            r = F.quantize(base, x[None, :])
            vals.append(F.scores(base, q[None, :], r["codes"], r["signs"], r["norms"], r["rnorms"])[0, 0])
        else:
            r = O.quantize(base, x[None, :])
            vals.append(O.scores(base, q[None, :], r["codes"], r["signs"], r["norms"], r["rnorms"])[0, 0])
    nu = np.linalg.norm(x)
    y = base.Pi @ (x / nu)
    if isinstance(base, F.FracParams):
        resid = y - base.centroids(F._codes_of(base, y[None, :]))[0]
    else:
        resid = y - base.c[np.searchsorted(base.t, y, side="left")]
    var = nu ** 2 * ((math.pi / 2) * (resid @ resid) * (q @ q) - (resid @ (base.Pi @ q)) ** 2) / d
    return np.array(vals), var, q @ x


def test_estimator_variance_closed_form_and_ordering():
    from dataclasses import replace
    d = 64
    vf, var_f, mean = _variance_over_S(lambda s: F.FracParams(d, 5, s))
    assert abs(vf.var(ddof=1) / var_f - 1) < 0.1
    assert abs(vf.mean() - mean) < 4 * math.sqrt(var_f / len(vf))
    v2, var2, _ = _variance_over_S(lambda s: replace(O.make_params(d, 2, s)))
    v3, var3, _ = _variance_over_S(lambda s: replace(O.make_params(d, 3, s)))
    # the same Pi in all three: 2.5 bits lies between 2 and 3 bits
    assert var3 < var_f < var2, (var3, var_f, var2)
    assert v3.var(ddof=1) < vf.var(ddof=1) < v2.var(ddof=1)


# ------------------------------------------------------------ planted mistakes
def test_planted_swapped_halves_are_caught(monkeypatch):
    orig = F.FracParams.centroids

    def swapped(self, idx):
        idx = np.asarray(idx)
        h = self.d // 2
        out = np.empty(idx.shape)
        out[:, :h] = self.c_lo[np.minimum(idx[:, :h], len(self.c_lo) - 1)]
        out[:, h:] = self.c_hi[idx[:, h:]]
        return out

    monkeypatch.setattr(F.FracParams, "centroids", swapped)
    with pytest.raises(AssertionError):
        test_each_half_is_coded_at_its_own_width(5)
    monkeypatch.setattr(F.FracParams, "centroids", orig)


def test_planted_floor_ceil_swap_and_plane_order_are_caught(monkeypatch):
    orig_init = F.FracParams.__init__

    def swapped_init(self, d, half_bits, seed, widths=None):
        orig_init(self, d, half_bits, seed, widths)
        if widths is None:
            self.w_hi, self.w_lo = self.w_lo, self.w_hi
            self.c_hi, self.t_hi, self.c_lo, self.t_lo = self.c_lo, self.t_lo, self.c_hi, self.t_hi

    monkeypatch.setattr(F.FracParams, "__init__", swapped_init)
    with pytest.raises(AssertionError):
        test_widths_of_the_two_settings()
    monkeypatch.setattr(F.FracParams, "__init__", orig_init)

    orig_pack = F.pack

    def reversed_planes(p, idx):
        flipped = np.asarray(idx).copy()
        h = p.d // 2
        flipped[:, :h] = ((flipped[:, :h] & 1) << 1) | ((flipped[:, :h] >> 1) & 1)
        return orig_pack(p, flipped)

    monkeypatch.setattr(F, "pack", reversed_planes)
    with pytest.raises(AssertionError):
        test_record_layout_hand_computed()
