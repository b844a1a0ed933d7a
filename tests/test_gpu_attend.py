"""GPU parity: tq_attend (fused decode attention over packed K and V)."""

import math

import numpy as np
import pytest

import oracle as O
from oblivious_kv_cache_amd import workloads as wl
from parity import assert_close

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from oblivious_kv_cache_amd import binding
    return binding


def _dev(rec, keys):
    return {k: torch.from_numpy(np.ascontiguousarray(rec[k])).cuda() for k in keys}


@pytest.mark.parametrize("d,kbits,vbits,G,qpg,T", [
    (128, 3, 3, 3, 4, 1000), (128, 3, 3, 1, 4, 512), (128, 3, 3, 2, 4, 513), (128, 2, 4, 2, 2, 777),
    (128, 4, 2, 1, 5, 300), (64, 3, 3, 2, 4, 1200), (128, 3, 3, 1, 4, 1), (96, 3, 1, 1, 8, 700),
    # every value width of the fused kernel at d = 128 and 64, and key widths at d = 64
    (128, 2, 1, 1, 4, 2000), (64, 4, 4, 2, 4, 700), (64, 2, 2, 1, 3, 1025), (64, 3, 1, 1, 4, 90),
    # several chunks per block (the value-record slots are refilled while a chunk is scored)
    (128, 3, 3, 64, 4, 8192), (128, 3, 4, 128, 4, 4096), (64, 3, 2, 64, 4, 8192),
    # lengths the fused kernel does not take (three steps)
    (32, 3, 3, 2, 4, 600),
])
def test_attend_matches_oracle(tq, d, kbits, vbits, G, qpg, T):
    pk = O.make_params(d, kbits, 0)
    pv = O.make_params(d, vbits, 1, "mse")
    K, _ = wl.outlier_keys_np(1, G, T, d, seed=4)
    K = K.reshape(G * T, d)
    V = wl.gaussian((G * T, d), 40)
    Q = wl.gaussian((G, qpg, d), 41)
    rk, rv = O.quantize(pk, K), O.quantize(pv, V)
    kctx, vctx = tq.Context(d, kbits, 0), tq.Context(d, vbits, 1, tq.TQ_MODE_MSE)
    scale = 1.0 / math.sqrt(d)
    print(f"attend d={d} kb={kbits} vb={vbits} G={G} qpg={qpg} T={T}", flush=True)
    out, logits, probs = tq.tq_attend(kctx, vctx, torch.from_numpy(Q).cuda(),
                                      _dev(rk, ("codes", "signs", "norms", "rnorms")),
                                      _dev(rv, ("codes", "norms")), scale, want_logits=True, want_probs=True)
    torch.cuda.synchronize()
    out, logits, probs = out.cpu().numpy(), logits.cpu().numpy(), probs.cpu().numpy()
    for g in range(G):
        sl = slice(g * T, (g + 1) * T)
        lw, pw, ow = O.attend(pk, pv, Q[g].astype(np.float64), rk["codes"][sl], rk["signs"][sl],
                              rk["norms"][sl], rk["rnorms"][sl], rv["codes"][sl], rv["norms"][sl], scale)
        assert_close(logits[g], lw, what=f"logits g{g}")
        assert_close(probs[g], pw, atol=1e-6, rtol=1e-3, what=f"probs g{g}")
        assert_close(out[g], ow, what=f"out g{g}")


def test_attend_unsupported_and_errors(tq):
    kctx, vctx = tq.Context(128, 3, 0), tq.Context(128, 3, 1, tq.TQ_MODE_MSE)
    q = torch.zeros((1, 4, 128), device="cuda")
    krec, vrec = kctx.empty_records(10), vctx.empty_records(10)
    with pytest.raises(tq.TQError):
        tq.tq_attend(vctx, kctx, q, krec, vrec, 0.1)          # roles swapped
    with pytest.raises(tq.TQError):
        tq.tq_attend(kctx, vctx, q, krec, vrec, 0.1, T=11, ldk=10)


def test_attend_128k_sampled(tq):
    """Long-context decode: 4 x 8 KV heads x 131072 tokens, d=128, K 3-bit
    TurboQuant, V 3-bit MSE-only, 32 query heads.  The whole cache is
    quantized on the GPU (sampled rows checked against the oracle); the
    records of two sampled groups are then replaced by the oracle's own
    encodings of the same rows, so the attention outputs of those groups can
    be compared exactly in the full-size launch."""
    from parity import check_quantized
    dev = torch.device("cuda")
    B, Hkv, T, d, Hq = 4, 8, 131072, 128, 32
    G, qpg = B * Hkv, Hq // Hkv
    kctx, vctx = tq.Context(d, 3, 0), tq.Context(d, 3, 1, tq.TQ_MODE_MSE)
    print("attend 128K: generating and quantizing K and V", flush=True)
    K, _ = wl.outlier_keys_torch(B, Hkv, T, d, seed=4, device=dev)
    V = wl.gaussian_torch((G * T, d), 44, dev, torch.bfloat16)
    krec = tq.tq_quantize(kctx, K.view(G * T, d))
    vrec = tq.tq_quantize(vctx, V)
    q = wl.gaussian_torch((B, Hq, d), 45, dev).view(G, qpg, d).contiguous()
    scale = 1.0 / math.sqrt(d)
    pk, pv = O.make_params(d, 3, 0), O.make_params(d, 3, 1, "mse")
    refs = {}
    rows = torch.arange(0, T, 97, device=dev)
    for g in (0, 17):
        Kg = K.view(G, T, d)[g].float().cpu().numpy()
        Vg = V.view(G, T, d)[g].float().cpu().numpy()
        rk, rv = O.quantize(pk, Kg, return_unpacked=True), O.quantize(pv, Vg, return_unpacked=True)
        r = rows.cpu().numpy()
        gk = {k: v.view(G, T, -1)[g][rows].cpu().numpy() for k, v in krec.items()}
        gk["norms"], gk["rnorms"] = gk["norms"].reshape(-1), gk["rnorms"].reshape(-1)
        sub = {k: v[r] for k, v in rk.items()}
        check_quantized(pk, gk, sub, Kg[r])
        for key in ("codes", "signs", "norms", "rnorms"):
            krec[key].view(G, T, -1)[g].copy_(torch.from_numpy(np.ascontiguousarray(rk[key])).view(T, -1))
        for key in ("codes", "norms"):
            vrec[key].view(G, T, -1)[g].copy_(torch.from_numpy(np.ascontiguousarray(rv[key])).view(T, -1))
        refs[g] = (rk, rv)
    out, logits, probs = tq.tq_attend(kctx, vctx, q, krec, vrec, scale, want_logits=True, want_probs=True)
    torch.cuda.synchronize()
    Q = q.cpu().numpy().astype(np.float64)
    for g, (rk, rv) in refs.items():
        lw, pw, ow = O.attend(pk, pv, Q[g], rk["codes"], rk["signs"], rk["norms"], rk["rnorms"],
                              rv["codes"], rv["norms"], scale)
        assert_close(logits[g].cpu().numpy(), lw, what=f"logits g{g}")
        assert_close(probs[g].cpu().numpy(), pw, atol=1e-7, rtol=1e-3, what=f"probs g{g}")
        assert_close(out[g].cpu().numpy(), ow, what=f"out g{g}")


def test_attend_deterministic(tq):
    # bitwise-identical repeats: split-K partials are combined in a fixed order
    d, G, qpg, T = 128, 3, 4, 5000
    kctx, vctx = tq.Context(d, 3, 0), tq.Context(d, 3, 1, tq.TQ_MODE_MSE)
    kc, ks, kn, kr = wl.random_records(G * T, kctx.code_bytes, kctx.sign_bytes, seed=60)
    vc, _, vn, _ = wl.random_records(G * T, vctx.code_bytes, 16, seed=61)
    krec = _dev({"codes": kc, "signs": ks, "norms": kn, "rnorms": kr}, ("codes", "signs", "norms", "rnorms"))
    vrec = _dev({"codes": vc, "norms": vn}, ("codes", "norms"))
    q = torch.from_numpy(wl.gaussian((G, qpg, d), 62)).cuda()
    runs = [tq.tq_attend(kctx, vctx, q, krec, vrec, 0.088, want_logits=True, want_probs=True) for _ in range(3)]
    torch.cuda.synchronize()
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert torch.equal(a, b)
