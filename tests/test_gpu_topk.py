"""GPU parity: tq_topk (fused estimator + top-k) against the oracle.

Acceptance with ties (several correct lists exist when scores tie within the
tolerance): at every rank r the oracle score of the GPU's id is within
tolerance of the oracle's r-th score, and the GPU and oracle id sets differ
only in ids whose oracle scores are within tolerance of the k-th score.
"""

import numpy as np
import pytest

import oracle as O
from oblivious_kv_cache_amd import workloads as wl
from parity import check_topk

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from oblivious_kv_cache_amd import binding
    return binding


def _setup(tq, d, bits, nq, n, seed, records="oracle"):
    p = O.make_params(d, bits, 0)
    ctx = tq.Context(d, bits, 0)
    if records == "oracle":
        X = wl.power_law(n, d, seed=seed, unit=True)
        rec = O.quantize(p, X)
    else:
        c, s, nu, g = wl.random_records(n, ctx.code_bytes, ctx.sign_bytes, seed)
        rec = {"codes": c, "signs": s, "norms": nu, "rnorms": g}
    Q = wl.power_law(nq, d, seed=seed + 1, unit=True)
    return p, ctx, rec, Q


def _run(tq, ctx, Q, rec, k):
    dev = torch.device("cuda")
    drec = {key: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for key, v in rec.items()}
    ids, sc = tq.tq_topk(ctx, torch.from_numpy(Q).to(dev), drec, k)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), sc.cpu().numpy()


@pytest.mark.parametrize("d,bits,nq,n,k", [
    (200, 2, 7, 1000, 10), (200, 4, 9, 1500, 10), (128, 3, 4, 777, 1), (128, 3, 5, 3000, 16),
    (200, 2, 3, 2000, 17), (64, 3, 6, 500, 64), (128, 2, 2, 64, 64), (200, 4, 1, 65, 10),
    # two query groups per scan wave, with an odd group count (the last wave's
    # second group is a repeat that must not be stored) and a ragged last group
    (128, 3, 9, 700, 10), (200, 2, 13, 900, 5),
])
def test_topk_matches_oracle(tq, d, bits, nq, n, k):
    p, ctx, rec, Q = _setup(tq, d, bits, nq, n, seed=d + n)
    print(f"topk d={d} b={bits} nq={nq} n={n} k={k}", flush=True)
    ids, sc = _run(tq, ctx, Q, rec, k)
    want = O.scores(p, Q.astype(np.float64), rec["codes"], rec["signs"], rec["norms"], rec["rnorms"])
    check_topk(ids, sc, want, k)


def test_topk_exact_ties_order_by_id(tq):
    d, bits = 128, 3
    p, ctx, rec, Q = _setup(tq, d, bits, 3, 200, seed=5)
    for key in rec:                       # rows 150..199 repeat rows 0..49: exact score ties
        rec[key] = rec[key].copy()
        rec[key][150:200] = rec[key][0:50]
    ids, sc = _run(tq, ctx, Q, rec, 20)
    for qi in range(3):
        for r in range(19):
            assert sc[qi, r] > sc[qi, r + 1] or (sc[qi, r] == sc[qi, r + 1] and ids[qi, r] < ids[qi, r + 1])
    want = O.scores(p, Q.astype(np.float64), rec["codes"], rec["signs"], rec["norms"], rec["rnorms"])
    check_topk(ids, sc, want, 20)


def test_topk_random_records_large_db(tq):
    d, bits, nq, n, k = 200, 2, 12, 200000, 10
    p, ctx, rec, Q = _setup(tq, d, bits, nq, n, seed=77, records="random")
    ids, sc = _run(tq, ctx, Q, rec, k)
    want = np.concatenate([O.scores(p, Q.astype(np.float64), rec["codes"][s:s + 50000], rec["signs"][s:s + 50000],
                                    rec["norms"][s:s + 50000], rec["rnorms"][s:s + 50000])
                           for s in range(0, n, 50000)], axis=1)
    check_topk(ids, sc, want, k)


@pytest.mark.parametrize("k", [10, 16])
def test_topk_pruning_with_mass_ties(tq, k):
    # 60000 records that are copies of 40 distinct ones: every lane sees many
    # exact ties of the best scores, so the pruning bound (the k-th best of
    # the lanes' current bests) equals real scores again and again; scores
    # equal to the bound must still enter, and ties resolve by lower id
    d, bits, nq, n = 128, 3, 5, 60000
    p, ctx, base, Q = _setup(tq, d, bits, nq, 40, seed=91, records="random")
    pick = np.random.default_rng(92).integers(0, 40, n)
    rec = {key: np.ascontiguousarray(v[pick]) for key, v in base.items()}
    ids, sc = _run(tq, ctx, Q, rec, k)
    want = O.scores(p, Q.astype(np.float64), rec["codes"], rec["signs"], rec["norms"], rec["rnorms"])
    check_topk(ids, sc, want, k)
    for qi in range(nq):                 # equal GPU scores come in increasing id order
        for r in range(k - 1):
            assert sc[qi, r] > sc[qi, r + 1] or (sc[qi, r] == sc[qi, r + 1] and ids[qi, r] < ids[qi, r + 1])


def test_topk_errors(tq):
    ctx = tq.Context(128, 3, 0)
    rec = ctx.empty_records(10)
    q = torch.zeros((2, 128), device="cuda")
    with pytest.raises(tq.TQError):
        tq.tq_topk(ctx, q, rec, 11)          # k > n
    with pytest.raises(tq.TQError):
        tq.tq_topk(ctx, q, rec, 1025)        # k > TQ_MAX_TOPK


@pytest.mark.parametrize("k", [10, 64])
def test_topk_deterministic(tq, k):
    # bitwise-identical repeats (ids and scores), including the candidate merge
    p, ctx, rec, Q = _setup(tq, 200, 2, 21, 30000, seed=77, records="random")
    a = _run(tq, ctx, Q, rec, k)
    b = _run(tq, ctx, Q, rec, k)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
