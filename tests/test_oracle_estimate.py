"""Pins for the oracle's softmax, value sum, top-k and recall."""

import numpy as np

import oracle as O


def test_softmax_properties():
    rng = np.random.default_rng(0)
    L = rng.standard_normal((5, 300)) * 20
    P = O.softmax(L, 0.125)
    assert np.allclose(P.sum(1), 1.0, atol=1e-14) and (P > 0).all()
    assert np.allclose(P, O.softmax(L + 17.0 / 0.125, 0.125), atol=1e-15)   # shift invariance
    # brute force on one row
    e = [np.exp(0.125 * v) for v in L[0]]
    assert np.allclose(P[0], np.array(e) / sum(e), rtol=1e-12)


def test_attend_is_probability_weighted_dequant_and_rotated_sum():
    d, T, qpg = 64, 200, 4
    pk = O.make_params(d, 3, 0)
    pv = O.make_params(d, 3, 1, "mse")
    rng = np.random.default_rng(1)
    K = rng.standard_normal((T, d))
    V = rng.standard_normal((T, d))
    Q = rng.standard_normal((qpg, d))
    rk, rv = O.quantize(pk, K), O.quantize(pv, V, return_unpacked=True)
    logits, probs, out = O.attend(pk, pv, Q, rk["codes"], rk["signs"], rk["norms"], rk["rnorms"],
                                  rv["codes"], rv["norms"], 1 / np.sqrt(d))
    assert np.allclose(logits, O.scores(pk, Q, rk["codes"], rk["signs"], rk["norms"], rk["rnorms"]))
    assert np.allclose(probs.sum(1), 1)
    # same result accumulated in the rotated domain, then rotated back once
    acc = probs @ (rv["norms"].astype(np.float64)[:, None] * pv.c[rv["idx"]])
    assert np.abs(acc @ pv.Pi - out).max() < 1e-12
    # explicit loop over tokens
    xh = O.dequant(pv, rv["codes"], None, rv["norms"], None)
    loop = sum(probs[:, t:t + 1] * xh[t][None, :] for t in range(T))
    assert np.abs(loop - out).max() < 1e-12


def test_topk_brute_force_with_ties():
    S = np.array([[0.5, 0.9, 0.9, 0.1, 0.9, -1.0],
                  [3.0, 2.0, 1.0, 0.0, -1.0, 4.0]])
    ids, vals = O.topk(S, 4)
    assert ids.tolist() == [[1, 2, 4, 0], [5, 0, 1, 2]]
    assert vals.tolist() == [[0.9, 0.9, 0.9, 0.5], [4.0, 3.0, 2.0, 1.0]]
    rng = np.random.default_rng(2)
    R = rng.integers(0, 20, (10, 50)).astype(float)      # many ties
    ids, _ = O.topk(R, 7)
    for i in range(10):
        ref = sorted(range(50), key=lambda j: (-R[i, j], j))[:7]
        assert ids[i].tolist() == ref


def test_exact_top1_and_recall():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((500, 16))
    Q = rng.standard_normal((40, 16))
    top1 = O.exact_top1(Q, X, chunk=7)
    assert np.array_equal(top1, np.argmax(Q @ X.T, axis=1))
    assert np.array_equal(O.exact_top1(Q, X, chunk=7, db_chunk=33), top1)   # chunked database
    X2 = np.vstack([X, X[:1]])                        # duplicate row -> tie, lower id wins
    assert (O.exact_top1(X[:1], X2) == 0).all()
    assert (O.exact_top1(X[:1], X2, db_chunk=100) == 0).all()   # the tie spans two chunks
    ids, _ = O.topk(Q @ X.T, 10)
    assert O.recall_at_k(ids, top1, 1) == 1.0
    noisy = Q @ X.T + rng.standard_normal((40, 500)) * 2
    ids, _ = O.topk(noisy, 10)
    rec = [O.recall_at_k(ids, top1, k) for k in (1, 2, 4, 8, 10)]
    assert rec == sorted(rec) and rec[0] < 1.0
