"""GPU parity: fractional bit widths (2.5 and 3.5 bits per coordinate) against
the oracle in oracle/frac.py -- quantize (codes and signs bit-exact outside
the 1e-5 decision band), the estimator (1e-4 + 1e-3 |oracle|) on the oracle's
own records and on generator records, reconstruction, and the calls that do
not take such a context."""

import numpy as np
import pytest

import oracle.frac as F
from oblivious_kv_cache_amd import workloads as wl
from parity import assert_close, check_quantized_frac

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from oblivious_kv_cache_amd import binding
    return binding


def _dev(rec, keys=("codes", "signs", "norms", "rnorms")):
    return {k: torch.from_numpy(np.ascontiguousarray(rec[k])).cuda() for k in keys}


def test_context_layout_and_codebooks(tq):
    for d, hb in [(128, 5), (128, 7), (256, 5), (256, 7)]:
        ctx = tq.Context(d, hb, 2, tq.TQ_MODE_FRAC)
        p = F.FracParams(d, hb, 2)
        assert (ctx.code_bytes, ctx.sign_bytes, ctx.w) == (p.code_bytes, p.sign_bytes, p.w_hi)
        Pi, S, (c1, c2), (t1, t2) = ctx.params()
        assert np.abs(Pi - p.Pi).max() < 1e-12 and np.abs(S - p.S).max() < 1e-12
        assert np.abs(c1 - p.c_hi).max() < 1e-13 and np.abs(c2 - p.c_lo).max() < 1e-13
        assert np.abs(t1 - p.t_hi).max() < 1e-13 and np.abs(t2 - p.t_lo).max() < 1e-13
    with pytest.raises(tq.TQError):
        tq.Context(64, 5, 0, tq.TQ_MODE_FRAC)


@pytest.mark.parametrize("d,hb,n,bf16", [
    (128, 5, 1000, False), (128, 7, 777, True), (256, 5, 301, True), (256, 7, 530, False), (128, 7, 17, False),
])
def test_quantize_frac(tq, d, hb, n, bf16):
    X = wl.outlier_keys_np(1, 1, n, d, seed=d + hb)[0].reshape(n, d)
    if bf16:
        X = wl.bf16_round(X)
    X[min(5, n - 1)] = 0.0
    print(f"quantize frac d={d} half_bits={hb} n={n} bf16={bf16}", flush=True)
    ctx = tq.Context(d, hb, 0, tq.TQ_MODE_FRAC)
    xt = torch.from_numpy(np.ascontiguousarray(X)).cuda()
    if bf16:
        xt = xt.to(torch.bfloat16)
    rec = tq.tq_quantize(ctx, xt)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in rec.items()}
    xin = xt.float().cpu().numpy()
    p = F.FracParams(d, hb, 0)
    print(check_quantized_frac(p, g, F.quantize(p, xin, return_unpacked=True), xin))


def test_quantize_frac_append_into_cache_slot(tq):
    # one new key per group into slot pos of a [G][ldk] cache: the slot's
    # record is 8-byte aligned (24-byte records)
    d, hb, G, ldk, pos = 128, 5, 6, 40, 17
    p = F.FracParams(d, hb, 0)
    ctx = tq.Context(d, hb, 0, tq.TQ_MODE_FRAC)
    cache = ctx.empty_records(G * ldk)
    X = wl.gaussian((G, d), 12)
    tq.tq_quantize(ctx, torch.from_numpy(X).cuda(), out={k: v[pos:] for k, v in cache.items()}, ldr=ldk)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in cache.items()}
    rows = np.arange(G) * ldk + pos
    check_quantized_frac(p, {k: v[rows] for k, v in g.items()}, F.quantize(p, X, return_unpacked=True), X)
    others = np.setdiff1d(np.arange(G * ldk), rows)
    assert not g["codes"][others].any() and not g["norms"][others].any()


def test_quantize_frac_strided_records(tq):
    d, hb, n = 128, 5, 70
    X = wl.gaussian((n, d), 3)
    ctx = tq.Context(d, hb, 1, tq.TQ_MODE_FRAC)
    rec = tq.tq_quantize(ctx, torch.from_numpy(X).cuda(), ldr=3)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in rec.items()}
    assert not g["codes"][1::3].any() and not g["norms"][2::3].any()     # records between are untouched
    g = {k: v[::3] for k, v in g.items()}
    p = F.FracParams(d, hb, 1)
    check_quantized_frac(p, g, F.quantize(p, X, return_unpacked=True), X)


def _oracle_grouped(p, Q, rec, G, T, ldk):
    return np.stack([F.scores(p, Q[g].astype(np.float64), rec["codes"][g * ldk:g * ldk + T],
                              rec["signs"][g * ldk:g * ldk + T], rec["norms"][g * ldk:g * ldk + T],
                              rec["rnorms"][g * ldk:g * ldk + T]) for g in range(G)])


@pytest.mark.parametrize("d,hb,G,qpg,T,ldk,records", [
    (128, 5, 3, 4, 1000, 1000, "oracle"), (128, 7, 2, 8, 513, 520, "oracle"), (128, 7, 1, 5, 300, 300, "random"),
    (256, 5, 2, 4, 257, 257, "random"), (256, 7, 1, 9, 700, 700, "oracle"), (128, 5, 2, 1, 1, 3, "random"),
    # group bases off 16 bytes (ldk * 24 and ldk * 40 odd multiples of 8): read lane by lane
    (128, 5, 3, 4, 400, 401, "random"), (128, 7, 2, 4, 333, 335, "oracle"),
])
def test_scores_frac(tq, d, hb, G, qpg, T, ldk, records):
    p = F.FracParams(d, hb, 0)
    ctx = tq.Context(d, hb, 0, tq.TQ_MODE_FRAC)
    if records == "oracle":
        rec = F.quantize(p, wl.outlier_keys_np(1, 1, G * ldk, d, seed=d)[0].reshape(G * ldk, d))
    else:
        c, s, nu, ga = wl.random_records(G * ldk, ctx.code_bytes, ctx.sign_bytes, seed=d + hb)
        rec = {"codes": c, "signs": s, "norms": nu, "rnorms": ga}
    Q = wl.gaussian((G, qpg, d), 21)
    print(f"scores frac d={d} half_bits={hb} G={G} qpg={qpg} T={T} ldk={ldk} {records}", flush=True)
    got = tq.tq_scores(ctx, torch.from_numpy(Q).cuda(), _dev(rec), T=T, ldk=ldk)
    static = tq.tq_scores_static(ctx, torch.from_numpy(Q).cuda(), _dev(rec), T=T, ldk=ldk)
    torch.cuda.synchronize()
    assert torch.equal(got, static)
    assert_close(got.cpu().numpy(), _oracle_grouped(p, Q, rec, G, T, ldk), what="logits")


@pytest.mark.parametrize("d,hb", [(128, 5), (256, 7)])
def test_dequant_frac(tq, d, hb):
    p = F.FracParams(d, hb, 5)
    X = wl.gaussian((60, d), 6)
    rec = F.quantize(p, X)
    ctx = tq.Context(d, hb, 5, tq.TQ_MODE_FRAC)
    out = tq.tq_dequant(ctx, _dev(rec)).cpu().numpy()
    want = F.dequant(p, rec["codes"], rec["signs"], rec["norms"], rec["rnorms"])
    scale = np.linalg.norm(want, axis=1, keepdims=True)
    assert (np.abs(out - want) <= 1e-5 * scale + 1e-6).all()


def test_frac_context_is_refused_where_unsupported(tq):
    kctx = tq.Context(128, 7, 0, tq.TQ_MODE_FRAC)
    vctx = tq.Context(128, 3, 1, tq.TQ_MODE_MSE)
    q = torch.zeros((1, 4, 128), device="cuda")
    krec, vrec = kctx.empty_records(64), vctx.empty_records(64)
    with pytest.raises(tq.TQError):
        tq.tq_attend(kctx, vctx, q, krec, vrec, 0.1)
    with pytest.raises(tq.TQError):
        tq.tq_topk(kctx, torch.zeros((2, 128), device="cuda"), krec, 5)
