"""Comparison rules shared by the GPU parity tests.

Acceptance (the precision contract of the hot path):
  * codes and sign bits are bit-exact, except a code whose oracle coordinate
    y_i lies within 1e-5 of a codebook threshold, or a sign whose oracle
    sketch value |z_j| < 1e-5 (unit-vector scale); such boundary mismatches
    must also stay below 1e-4 of all codes (signs counted separately);
  * norms nu: within 1 float32 ulp of the float64 length;
  * residual norms gamma (vectors whose codes all match): |diff| <= 2e-5 +
    1e-5 * gamma (the GPU's rotated coordinates carry ~1e-6 absolute error per
    coordinate, and |d gamma| <= |d y|_2);
  * floating-point outputs (logits, probabilities, reconstructions):
    |gpu - oracle| <= 1e-4 + 1e-3 * |oracle|, with the oracle evaluated on the
    same inputs the GPU consumed (oracle-made records or generator data).
"""

import numpy as np

import oracle as O

BAND = 1e-5
MAX_FRAC = 1e-4
ATOL, RTOL = 1e-4, 1e-3


def assert_close(got, want, atol=ATOL, rtol=RTOL, what="values"):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    excess = np.abs(got - want) - (atol + rtol * np.abs(want))
    bad = excess > 0
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst excess "
                           f"{excess.max():.3e} at {np.unravel_index(np.argmax(excess), excess.shape)}")


def check_quantized(p, gpu, ref, X=None, allow_frac=MAX_FRAC):
    """Compare GPU records with the oracle's (``ref`` from quantize(return_unpacked=True)).

    A vector whose code differs inside the band has two valid encodings; its
    sign bits and gamma are then checked against the oracle's stage-2 result
    for the other valid code choice (needs the input rows ``X``).
    """
    g_idx = O.unpack_codes(p, gpu["codes"])
    r_idx = ref["idx"]
    assert np.array_equal(gpu["codes"].shape, ref["codes"].shape)
    # norms: within one float32 ulp of the float64 length
    gn, rn = gpu["norms"].astype(np.float32), ref["norms"].astype(np.float32)
    assert (np.abs(gn.astype(np.float64) - rn) <= np.spacing(np.maximum(np.abs(rn), 1e-30))).all()
    # codes
    diff = g_idx != r_idx
    if diff.any():
        y = ref["y"][diff]
        dist = np.min(np.abs(y[:, None] - p.t[None, :]), axis=1)
        assert (dist < BAND).all(), f"code mismatch outside the band: min dist {dist.max():.3e}"
        # the GPU's code must be the neighbour across that threshold
        assert (np.abs(g_idx[diff] - r_idx[diff]) == 1).all()
    assert diff.sum() <= allow_frac * diff.size, f"{diff.sum()} code mismatches of {diff.size}"
    bits = np.unpackbits(gpu["codes"], axis=1, bitorder="little")
    assert not bits[:, p.w * p.d:].any(), "nonzero code padding"
    stats = {"code_mismatch": int(diff.sum())}
    if p.mode == "prod":
        g_s = O.unpack_bits(gpu["signs"], 1, p.m)
        z_ref = ref["z"].copy()
        s_ref = ref["sbits"].copy()
        g_ref = ref["rnorms"].astype(np.float64).copy()
        for v in np.nonzero(diff.any(axis=1))[0]:
            assert X is not None, "input rows needed to check a vector with a boundary code"
            alt = r_idx[v].copy()
            alt[diff[v]] = g_idx[v][diff[v]]          # the other valid side of each tied coordinate
            gam, z, sb = O.stage2_from_codes(p, X[v], alt)
            z_ref[v], s_ref[v], g_ref[v] = z, sb, gam
        sdiff = g_s != s_ref
        if sdiff.any():
            z = np.abs(z_ref[sdiff])
            assert (z < BAND).all(), f"sign mismatch outside the band: |z| {z.max():.3e}"
        assert sdiff.sum() <= allow_frac * sdiff.size, f"{sdiff.sum()} sign mismatches"
        sb = np.unpackbits(gpu["signs"], axis=1, bitorder="little")
        assert not sb[:, p.m:].any(), "nonzero sign padding"
        stats["sign_mismatch"] = int(sdiff.sum())
        gg = gpu["rnorms"].astype(np.float64)
        assert (np.abs(gg - g_ref) <= 2e-5 + 1e-5 * g_ref).all(), np.abs(gg - g_ref).max()
    zero = ref["norms"] == 0
    if zero.any():
        assert not gpu["codes"][zero].any()
        if p.mode == "prod":
            assert not gpu["signs"][zero].any() and (gpu["rnorms"][zero] == 0).all()
    return stats


# Top-k lists.  Several correct lists exist when scores tie within the
# tolerance: at every rank r the oracle score of the GPU's id must be within
# tolerance of the oracle's r-th score, and the GPU and oracle id sets may
# differ only in ids whose oracle scores are within tolerance of the k-th.
TK_ATOL, TK_RTOL = 1e-4, 1e-3


def check_topk(gpu_ids, gpu_scores, oracle_scores, k):
    """oracle_scores: [nq, n] float64 oracle estimator scores."""
    ref_ids, ref_vals = O.topk(oracle_scores, k)
    for qi in range(len(gpu_ids)):
        g = gpu_ids[qi]
        assert len(set(g.tolist())) == k, "duplicate ids"
        sc = oracle_scores[qi]
        tol = TK_ATOL + TK_RTOL * np.abs(ref_vals[qi])
        assert (np.abs(sc[g] - ref_vals[qi]) <= tol).all(), (qi, sc[g] - ref_vals[qi])
        assert (np.abs(gpu_scores[qi] - sc[g]) <= TK_ATOL + TK_RTOL * np.abs(sc[g])).all()
        kth = ref_vals[qi][-1]
        for i in set(g.tolist()) ^ set(ref_ids[qi].tolist()):
            assert abs(sc[i] - kth) <= TK_ATOL + TK_RTOL * abs(kth), (qi, i, sc[i], kth)


def check_polar(p, gpu, X, allow_frac=MAX_FRAC):
    """PolarQuant records against the oracle (oracle/polar.py): norms within one
    float32 ulp; slot codes bit-exact except an angle whose rotated point lies
    within 1e-5 (unit-sphere scale) of a decision boundary of its level (then
    the neighbouring code, or across the 0 = 2 pi wrap at level 1), such
    slots below 1e-4 of all; the spare slot of quarter 3 and the padding zero."""
    import oracle.polar as PQ
    ref = PQ.quantize(p, X)
    g_idx = O.unpack_bits(gpu["codes"], p.bits, p.d)
    gn, rn = gpu["norms"].astype(np.float32), ref["norms"].astype(np.float32)
    assert (np.abs(gn.astype(np.float64) - rn) <= np.spacing(np.maximum(np.abs(rn), 1e-30))).all()
    diff = g_idx != ref["idx"]
    n = 2 ** p.bits
    for v, s in zip(*np.nonzero(diff)):
        m = PQ.slot_margins(p, X[v])[s]
        assert m < BAND, f"vector {v} slot {s}: code {g_idx[v, s]} vs {ref['idx'][v, s]}, margin {m:.3e}"
        dist = abs(int(g_idx[v, s]) - int(ref["idx"][v, s]))
        assert dist == 1 or dist == n - 1, (v, s, dist)
    assert diff.sum() <= allow_frac * diff.size, f"{diff.sum()} angle-code mismatches of {diff.size}"
    bits = np.unpackbits(gpu["codes"], axis=1, bitorder="little")
    assert not bits[:, p.bits * p.d:].any(), "nonzero code padding"
    assert not g_idx[:, p.d - 1].any(), "spare slot of the last quarter"
    zero = ref["norms"] == 0
    assert not gpu["codes"][zero].any()
    return int(diff.sum())


def check_quantized_frac(p, gpu, ref, X, allow_frac=MAX_FRAC):
    """Fractional-width records (oracle/frac.py) against the oracle's: the rules
    of check_quantized, with each coordinate's thresholds those of its half."""
    import oracle.frac as F
    g_idx, r_idx = F.unpack(p, gpu["codes"]), ref["idx"]
    assert gpu["codes"].shape == ref["codes"].shape
    gn, rn = gpu["norms"].astype(np.float32), ref["norms"].astype(np.float32)
    assert (np.abs(gn.astype(np.float64) - rn) <= np.spacing(np.maximum(np.abs(rn), 1e-30))).all()
    diff = g_idx != r_idx
    h = p.d // 2
    for v, i in zip(*np.nonzero(diff)):
        t = p.t_hi if i < h else p.t_lo
        dist = np.min(np.abs(ref["y"][v, i] - t))
        assert dist < BAND, f"vector {v} coordinate {i}: code mismatch outside the band ({dist:.3e})"
        assert abs(int(g_idx[v, i]) - int(r_idx[v, i])) == 1
    assert diff.sum() <= allow_frac * diff.size, f"{diff.sum()} code mismatches of {diff.size}"
    g_s = O.unpack_bits(gpu["signs"], 1, p.m)
    z_ref, s_ref = ref["z"].copy(), ref["sbits"].copy()
    g_ref = ref["rnorms"].astype(np.float64).copy()
    for v in np.nonzero(diff.any(axis=1))[0]:
        alt = r_idx[v].copy()
        alt[diff[v]] = g_idx[v][diff[v]]
        g_ref[v], z_ref[v], s_ref[v] = F.stage2_from_codes(p, X[v], alt)
    sdiff = g_s != s_ref
    if sdiff.any():
        z = np.abs(z_ref[sdiff])
        assert (z < BAND).all(), f"sign mismatch outside the band: |z| {z.max():.3e}"
    assert sdiff.sum() <= allow_frac * sdiff.size, f"{sdiff.sum()} sign mismatches"
    assert not np.unpackbits(gpu["signs"], axis=1, bitorder="little")[:, p.m:].any(), "nonzero sign padding"
    gg = gpu["rnorms"].astype(np.float64)
    assert (np.abs(gg - g_ref) <= 2e-5 + 1e-5 * g_ref).all(), np.abs(gg - g_ref).max()
    zero = ref["norms"] == 0
    if zero.any():
        assert not gpu["codes"][zero].any() and not gpu["signs"][zero].any()
        assert (gpu["rnorms"][zero] == 0).all()
    return {"code_mismatch": int(diff.sum()), "sign_mismatch": int(sdiff.sum())}
