"""GPU parity for vectors longer than 256 coordinates (d up to 1024) and top-k
lists longer than 64 (k up to 1024): the kernels that stage vectors and
operand fragments in LDS and walk records of any length in a runtime loop.

Sizes span several 16-vector / 64-key tiles with ragged tails; the oracle
evaluates the same records the GPU reads (its own encodings, or generator
records).
"""

import math

import numpy as np
import pytest

import oracle as O
from oblivious_kv_cache_amd import workloads as wl
from parity import assert_close, check_quantized, check_topk

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from oblivious_kv_cache_amd import binding
    return binding


def _dev(rec, keys=None):
    keys = keys or rec.keys()
    return {k: torch.from_numpy(np.ascontiguousarray(rec[k])).cuda() for k in keys}


@pytest.mark.parametrize("d,bits,n,bf16", [
    (264, 2, 301, False), (512, 3, 257, False), (512, 4, 333, True), (1024, 2, 97, True),
    (1024, 3, 130, False), (1024, 4, 65, True), (1016, 3, 50, False),
])
def test_quantize_large_d(tq, d, bits, n, bf16):
    X = wl.outlier_keys_np(1, 1, n, d, seed=d + bits)[0].reshape(n, d)
    if bf16:
        X = wl.bf16_round(X)
    print(f"quantize d={d} b={bits} n={n} bf16={bf16}", flush=True)
    ctx = tq.Context(d, bits, 0)
    xt = torch.from_numpy(np.ascontiguousarray(X)).cuda()
    if bf16:
        xt = xt.to(torch.bfloat16)
    rec = tq.tq_quantize(ctx, xt)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in rec.items()}
    xin = xt.float().cpu().numpy()
    p = O.make_params(d, bits, 0)
    check_quantized(p, g, O.quantize(p, xin, return_unpacked=True), xin)


@pytest.mark.parametrize("d,bits", [(520, 1), (1024, 4)])
def test_quantize_large_d_mse(tq, d, bits):
    n = 200
    X = wl.gaussian((n, d), 5)
    ctx = tq.Context(d, bits, 3, tq.TQ_MODE_MSE)
    rec = tq.tq_quantize(ctx, torch.from_numpy(X).cuda())
    torch.cuda.synchronize()
    g = {k: (v.cpu().numpy() if v is not None else None) for k, v in rec.items()}
    p = O.make_params(d, bits, 3, "mse")
    check_quantized(p, g, O.quantize(p, X, return_unpacked=True), X)


def test_quantize_large_d_zero_tiny_and_strided(tq):
    d, bits, n = 520, 3, 40
    X = wl.gaussian((n, d), 8)
    X[3] = 0.0
    X[17] *= 1e-30                     # below 2^-64: rescaled before the rotation
    X[20] *= 1e-39
    ctx = tq.Context(d, bits, 0)
    xs = torch.zeros((n, d + 24), device="cuda")
    xs[:, :d] = torch.from_numpy(X).cuda()
    rec = tq.tq_quantize(ctx, xs[:, :d], ldr=2)        # strided input, every other record
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy()[::2][:n] for k, v in rec.items()}
    p = O.make_params(d, bits, 0)
    xin = xs[:, :d].cpu().numpy()
    check_quantized(p, g, O.quantize(p, xin, return_unpacked=True), xin)
    assert g["norms"][3] == 0 and not g["codes"][3].any() and not g["signs"][3].any()


@pytest.mark.parametrize("mode,bits,d", [("prod", 3, 512), ("mse", 2, 1024), ("prod", 4, 1024)])
def test_dequant_large_d(tq, mode, bits, d):
    n = 37
    X = wl.gaussian((n, d), 9)
    p = O.make_params(d, bits, 1, mode)
    rec = O.quantize(p, X)
    ctx = tq.Context(d, bits, 1, tq.TQ_MODE_PROD if mode == "prod" else tq.TQ_MODE_MSE)
    keys = ("codes", "signs", "norms", "rnorms") if mode == "prod" else ("codes", "norms")
    out = tq.tq_dequant(ctx, _dev(rec, keys)).cpu().numpy()
    want = O.dequant(p, rec["codes"], rec["signs"], rec["norms"], rec["rnorms"])
    scale = np.linalg.norm(want, axis=1, keepdims=True)
    assert (np.abs(out - want) <= 1e-5 * scale + 1e-6).all()


@pytest.mark.parametrize("d,bits,G,qpg,T,ldk,records", [
    (264, 2, 2, 4, 300, 300, "oracle"), (512, 3, 1, 5, 257, 260, "oracle"), (512, 4, 2, 4, 129, 129, "random"),
    (1024, 2, 1, 8, 200, 200, "random"), (1024, 4, 2, 3, 191, 200, "oracle"), (1000, 4, 1, 4, 65, 65, "random"),
    (768, 3, 1, 1, 1, 1, "random"),
])
def test_scores_large_d(tq, d, bits, G, qpg, T, ldk, records):
    ctx = tq.Context(d, bits, 0)
    p = O.make_params(d, bits, 0)
    if records == "oracle":
        rec = O.quantize(p, wl.gaussian((G * ldk, d), d + 1))
    else:
        c, s, nu, ga = wl.random_records(G * ldk, ctx.code_bytes, ctx.sign_bytes, seed=d + bits)
        rec = {"codes": c, "signs": s, "norms": nu, "rnorms": ga}
    Q = wl.gaussian((G, qpg, d), 21)
    print(f"scores d={d} b={bits} G={G} qpg={qpg} T={T} ldk={ldk} {records}", flush=True)
    got = tq.tq_scores(ctx, torch.from_numpy(Q).cuda(), _dev(rec), T=T, ldk=ldk)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    for g in range(G):
        sl = slice(g * ldk, g * ldk + T)
        want = O.scores(p, Q[g].astype(np.float64), rec["codes"][sl], rec["signs"][sl], rec["norms"][sl],
                        rec["rnorms"][sl])
        assert_close(got[g], want, what=f"logits g{g}")


def test_scores_large_d_extreme_query(tq):
    # one coordinate dominates the query: the digit scale follows it, and
    # every other coefficient is carried by the lower digits
    d, bits, T = 1024, 4, 300
    ctx, p = tq.Context(d, bits, 0), O.make_params(d, bits, 0)
    rec = O.quantize(p, wl.gaussian((T, d), 3))
    Q = wl.gaussian((1, 4, d), 4)
    Q[0, 0, 5] = 1e4
    Q[0, 1] *= 1e-20
    got = tq.tq_scores(ctx, torch.from_numpy(Q).cuda(), _dev(rec)).cpu().numpy()
    want = O.scores(p, Q[0].astype(np.float64), rec["codes"], rec["signs"], rec["norms"], rec["rnorms"])
    assert_close(got[0, 0], want[0], atol=1e-4 * np.abs(want[0]).max(), what="dominant coordinate")
    assert_close(got[0, 2:], want[2:], what="ordinary heads")
    assert_close(got[0, 1], want[1], atol=1e-24, what="tiny head")


@pytest.mark.parametrize("d,bits,nq,n,k", [
    (200, 2, 5, 3000, 100), (128, 3, 3, 2500, 1024), (512, 3, 6, 1500, 10), (1024, 4, 2, 1100, 100),
    (264, 2, 9, 700, 65), (128, 4, 1, 1024, 1024),
])
def test_topk_large_k_and_d(tq, d, bits, nq, n, k):
    p, ctx = O.make_params(d, bits, 0), tq.Context(d, bits, 0)
    X = wl.power_law(n, d, seed=d + n, unit=True)
    rec = O.quantize(p, X)
    Q = wl.power_law(nq, d, seed=d + n + 1, unit=True)
    print(f"topk d={d} b={bits} nq={nq} n={n} k={k}", flush=True)
    ids, sc = tq.tq_topk(ctx, torch.from_numpy(Q).cuda(), _dev(rec), k)
    torch.cuda.synchronize()
    want = O.scores(p, Q.astype(np.float64), rec["codes"], rec["signs"], rec["norms"], rec["rnorms"])
    check_topk(ids.cpu().numpy(), sc.cpu().numpy(), want, k)


def test_topk_large_k_mass_ties_and_determinism(tq):
    # 20000 records drawn from 300 distinct ones: many exact ties at the list
    # threshold; ties order by id, and repeats are bitwise identical
    d, bits, nq, n, k = 128, 3, 5, 20000, 200
    ctx, p = tq.Context(d, bits, 0), O.make_params(d, bits, 0)
    c, s, nu, ga = wl.random_records(300, ctx.code_bytes, ctx.sign_bytes, 93)
    pick = np.random.default_rng(94).integers(0, 300, n)
    rec = {"codes": c[pick], "signs": s[pick], "norms": nu[pick], "rnorms": ga[pick]}
    Q = wl.power_law(nq, d, seed=95, unit=True)
    dq, drec = torch.from_numpy(Q).cuda(), _dev(rec)
    runs = [tq.tq_topk(ctx, dq, drec, k) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])
    ids, sc = runs[0][0].cpu().numpy(), runs[0][1].cpu().numpy()
    for qi in range(nq):
        for r in range(k - 1):
            assert sc[qi, r] > sc[qi, r + 1] or (sc[qi, r] == sc[qi, r + 1] and ids[qi, r] < ids[qi, r + 1])
    want = O.scores(p, Q.astype(np.float64), rec["codes"], rec["signs"], rec["norms"], rec["rnorms"])
    check_topk(ids, sc, want, k)


@pytest.mark.parametrize("d,kbits,vbits,G,qpg,T", [
    (256, 3, 3, 2, 4, 1000), (256, 2, 4, 1, 5, 777), (512, 4, 2, 2, 3, 513), (1024, 3, 1, 1, 4, 300),
    (136, 3, 3, 1, 8, 600), (1024, 4, 4, 1, 2, 1),
])
def test_attend_large_d(tq, d, kbits, vbits, G, qpg, T):
    pk = O.make_params(d, kbits, 0)
    pv = O.make_params(d, vbits, 1, "mse")
    K = wl.outlier_keys_np(1, G, T, d, seed=4)[0].reshape(G * T, d)
    V = wl.gaussian((G * T, d), 40)
    Q = wl.gaussian((G, qpg, d), 41)
    rk, rv = O.quantize(pk, K), O.quantize(pv, V)
    kctx, vctx = tq.Context(d, kbits, 0), tq.Context(d, vbits, 1, tq.TQ_MODE_MSE)
    scale = 1.0 / math.sqrt(d)
    print(f"attend d={d} kb={kbits} vb={vbits} G={G} qpg={qpg} T={T}", flush=True)
    kd, vd = _dev(rk, ("codes", "signs", "norms", "rnorms")), _dev(rv, ("codes", "norms"))
    out, logits, probs = tq.tq_attend(kctx, vctx, torch.from_numpy(Q).cuda(), kd, vd, scale,
                                      want_logits=True, want_probs=True)
    out_only = tq.tq_attend(kctx, vctx, torch.from_numpy(Q).cuda(), kd, vd, scale)[0]
    torch.cuda.synchronize()
    assert torch.equal(out, out_only)           # logits in the workspace or in the output: same result
    out, logits, probs = out.cpu().numpy(), logits.cpu().numpy(), probs.cpu().numpy()
    for g in range(G):
        sl = slice(g * T, (g + 1) * T)
        lw, pw, ow = O.attend(pk, pv, Q[g].astype(np.float64), rk["codes"][sl], rk["signs"][sl],
                              rk["norms"][sl], rk["rnorms"][sl], rv["codes"][sl], rv["norms"][sl], scale)
        assert_close(logits[g], lw, what=f"logits g{g}")
        assert_close(probs[g], pw, atol=1e-6, rtol=1e-3, what=f"probs g{g}")
        assert_close(out[g], ow, what=f"out g{g}")
