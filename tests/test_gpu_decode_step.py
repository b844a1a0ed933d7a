"""GPU parity: tq_decode_step (append the new key and value, then attend)."""

import math

import numpy as np
import pytest

import oracle as O
from oblivious_kv_cache_amd import workloads as wl
from parity import assert_close

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MARGIN = 1e-4     # new tokens are drawn clear of every decision boundary


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from oblivious_kv_cache_amd import binding
    return binding


def _clear_rows(p, G, d, seed, bf16):
    """G vectors whose oracle encoding has no coordinate within MARGIN of a
    threshold and no sketch value within MARGIN of 0 (so the encoding is
    unique and the GPU must reproduce it bit for bit).  Rows are redrawn
    from successive seeds until clear."""
    rows, s = [], seed
    while len(rows) < G:
        x = wl.gaussian((1, d), s)
        if bf16:
            x = wl.bf16_round(x)
        r = O.quantize(p, x.astype(np.float64), return_unpacked=True)
        dist = np.min(np.abs(r["y"][0][:, None] - p.t[None, :]))
        zmin = np.min(np.abs(r["z"][0])) if r["z"].size else 1.0
        if dist > MARGIN and zmin > MARGIN:
            rows.append(x[0])
        s += 1
    return np.stack(rows)


# d = 128 with equal key/value bits takes the one-launch append + prep; d = 64
# and mixed bit widths take the separate launches
@pytest.mark.parametrize("d,kb,vb,G,qpg,ldk,pos,bf16", [
    (128, 3, 3, 3, 4, 700, 600, False), (128, 3, 3, 2, 4, 1100, 1024, True), (128, 3, 3, 2, 3, 64, 0, False),
    (128, 3, 3, 1, 8, 520, 511, True), (128, 4, 4, 2, 4, 300, 299, True), (128, 2, 2, 3, 4, 90, 50, False),
    (64, 3, 3, 2, 4, 600, 555, False), (128, 3, 2, 2, 4, 400, 123, True),
    # longer vectors: logits, value sum and combine in three steps
    (256, 3, 3, 2, 4, 300, 257, True), (512, 4, 2, 1, 5, 200, 130, False)])
def test_decode_step_matches_oracle(tq, d, kb, vb, G, qpg, ldk, pos, bf16):
    pk, pv = O.make_params(d, kb, 0), O.make_params(d, vb, 1, "mse")
    kctx, vctx = tq.Context(d, kb, 0), tq.Context(d, vb, 1, tq.TQ_MODE_MSE)
    K = wl.gaussian((G * ldk, d), 70)
    V = wl.gaussian((G * ldk, d), 71)
    rk, rv = O.quantize(pk, K), O.quantize(pv, V)
    newk = _clear_rows(pk, G, d, 1000, bf16)
    newv = _clear_rows(pv, G, d, 2000, bf16)
    ek, ev = O.quantize(pk, newk.astype(np.float64)), O.quantize(pv, newv.astype(np.float64))
    Q = wl.gaussian((G, qpg, d), 72)
    dev = torch.device("cuda")
    krec = {k: torch.from_numpy(np.ascontiguousarray(rk[k])).to(dev) for k in ("codes", "signs", "norms", "rnorms")}
    vrec = {k: torch.from_numpy(np.ascontiguousarray(rv[k])).to(dev) for k in ("codes", "norms")}
    before = {k: v.clone() for k, v in krec.items()}
    vbefore = {k: v.clone() for k, v in vrec.items()}
    dt = torch.bfloat16 if bf16 else torch.float32
    nk = torch.from_numpy(newk.astype(np.float32)).to(dev).to(dt)
    nv = torch.from_numpy(newv.astype(np.float32)).to(dev).to(dt)
    scale = 1.0 / math.sqrt(d)
    print(f"decode step d={d} kb={kb} vb={vb} G={G} qpg={qpg} ldk={ldk} pos={pos} bf16={bf16}", flush=True)
    out, logits, probs = tq.tq_decode_step(kctx, vctx, torch.from_numpy(Q).to(dev), nk, nv, krec, vrec,
                                           pos, scale, ldk=ldk, want_logits=True, want_probs=True)
    torch.cuda.synchronize()
    slots = [g * ldk + pos for g in range(G)]
    # the appended records are the oracle's (bit for bit; norms within 1 ulp)
    for k in ("codes", "signs"):
        assert np.array_equal(krec[k][slots].cpu().numpy(), ek[k]), k
    assert np.array_equal(vrec["codes"][slots].cpu().numpy(), ev["codes"])
    for got, want in ((krec["norms"][slots], ek["norms"]), (vrec["norms"][slots], ev["norms"])):
        got = got.cpu().numpy().astype(np.float64)
        assert (np.abs(got - want) <= np.spacing(np.abs(want).astype(np.float32))).all()
    assert np.allclose(krec["rnorms"][slots].cpu().numpy(), ek["rnorms"], rtol=1e-5, atol=2e-5)
    # every other record is untouched
    mask = torch.ones(G * ldk, dtype=torch.bool, device=dev)
    mask[slots] = False
    for k in krec:
        assert torch.equal(krec[k][mask], before[k][mask]), k
    for k in vrec:
        assert torch.equal(vrec[k][mask], vbefore[k][mask]), k
    # attention over tokens 0..pos with the oracle's records throughout
    for k in ("codes", "signs", "norms", "rnorms"):
        rk[k][slots] = ek[k]
    for k in ("codes", "norms"):
        rv[k][slots] = ev[k]
    for g in range(G):
        sl = slice(g * ldk, g * ldk + pos + 1)
        lw, pw, ow = O.attend(pk, pv, Q[g].astype(np.float64), rk["codes"][sl], rk["signs"][sl], rk["norms"][sl],
                              rk["rnorms"][sl], rv["codes"][sl], rv["norms"][sl], scale)
        assert_close(logits[g].cpu().numpy(), lw, what=f"logits g{g}")
        assert_close(probs[g].cpu().numpy(), pw, atol=1e-6, rtol=1e-3, what=f"probs g{g}")
        assert_close(out[g].cpu().numpy(), ow, what=f"out g{g}")


def test_decode_step_rejects_before_writing(tq):
    d = 128
    kctx, vctx = tq.Context(d, 3, 0), tq.Context(d, 3, 1, tq.TQ_MODE_MSE)
    dev = torch.device("cuda")
    krec, vrec = kctx.empty_records(2 * 16, dev), vctx.empty_records(2 * 16, dev)
    q = torch.zeros((2, 4, d), device=dev)
    nk = torch.ones((2, d), device=dev)
    with pytest.raises(tq.TQError):        # pos past the cache
        tq.tq_decode_step(kctx, vctx, q, nk, nk, krec, vrec, 16, 0.1, ldk=16)
    with pytest.raises(tq.TQError):        # contexts swapped
        tq.tq_decode_step(vctx, kctx, q, nk, nk, krec, vrec, 3, 0.1, ldk=16)
    torch.cuda.synchronize()
    assert not krec["codes"].any() and not krec["norms"].any() and not vrec["codes"].any()


@pytest.mark.parametrize("d,bits,with_v", [(128, 3, True), (128, 3, False), (128, 2, True), (64, 3, False)])
def test_decode_prep_matches_separate_calls(tq, d, bits, with_v):
    """tq_decode_prep (one launch at d = 128) writes exactly what tq_quantize
    and tq_prep_queries write, and scoring the prepared workspace over T =
    pos + 1 tokens equals tq_scores on the updated cache."""
    G, qpg, ldk, pos = 5, 4, 300, 211
    dev = torch.device("cuda")
    kctx = tq.Context(d, bits, 0)
    vctx = tq.Context(d, bits, 1, tq.TQ_MODE_MSE) if with_v else None
    kc, ks, kn, kr = wl.random_records(G * ldk, kctx.code_bytes, kctx.sign_bytes, seed=80)
    krec = {"codes": kc, "signs": ks, "norms": kn, "rnorms": kr}
    krec = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in krec.items()}
    vrec = None
    if with_v:
        vc_, _, vn, _ = wl.random_records(G * ldk, vctx.code_bytes, 16, seed=81)
        vrec = {"codes": torch.from_numpy(vc_).to(dev), "norms": torch.from_numpy(vn).to(dev)}
    nk = torch.from_numpy(wl.bf16_round(wl.gaussian((G, d), 82))).to(dev).to(torch.bfloat16)
    nv = torch.from_numpy(wl.bf16_round(wl.gaussian((G, d), 83))).to(dev).to(torch.bfloat16)
    q = torch.from_numpy(wl.gaussian((G, qpg, d), 84)).to(dev)
    k2 = {k: v.clone() for k, v in krec.items()}
    v2 = {k: v.clone() for k, v in vrec.items()} if with_v else None
    print(f"decode prep d={d} b={bits} values={with_v}", flush=True)
    ws = tq.tq_decode_prep(kctx, q, nk, krec, pos, ldk=ldk, vctx=vctx, new_v=nv if with_v else None, vrec=vrec)
    tq.tq_quantize(kctx, nk, out={k: v[pos:] for k, v in k2.items()}, ldr=ldk)
    if with_v:
        tq.tq_quantize(vctx, nv, out={"codes": v2["codes"][pos:], "signs": None, "norms": v2["norms"][pos:],
                                      "rnorms": None}, ldr=ldk)
    ws2 = tq.tq_prep_queries(kctx, q)
    torch.cuda.synchronize()
    for k in krec:
        assert torch.equal(krec[k], k2[k]), k
    if with_v:
        for k in vrec:
            assert torch.equal(vrec[k], v2[k]), k
    # the prepared state of every (group, 4-head block): NM operand fragments
    # of 1 KB and 64 B of constants, in 256-byte-aligned strides
    cb16, sb16, w = kctx.code_bytes // 16, kctx.sign_bytes // 16, kctx.w
    nm = 2 * cb16 + (2 * cb16 if w == 3 else 0) + 2 * sb16
    used, stride = nm * 1024 + 64, (nm * 1024 + 64 + 255) // 256 * 256
    ngroups = G * ((qpg + 3) // 4)
    a = ws[:ngroups * stride].view(ngroups, stride)[:, :used]
    b = ws2[:ngroups * stride].view(ngroups, stride)[:, :used]
    assert torch.equal(a, b)
    T = pos + 1
    got = tq.tq_scores_prepared(kctx, ws, G, qpg, krec, T=T, ldk=ldk)
    ref = tq.tq_scores(kctx, q, k2, T=T, ldk=ldk)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
