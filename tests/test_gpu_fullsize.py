"""GPU parity at full workload size, on sampled outputs.

Decode at 32K context: 32 x 8 KV heads x 32768 tokens x d=128 bf16 keys (4
outlier channels per head), 32 query heads, b = 3 and 4, in the launch
configuration bench.py times.  The whole cache is quantized and scored on the
GPU; the oracle then quantizes a sample of the same key rows itself and
recomputes the logits of those keys one by one.
"""

import math

import numpy as np
import pytest

import oracle as O
from oblivious_kv_cache_amd import workloads as wl
from parity import assert_close, check_quantized

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from oblivious_kv_cache_amd import binding
    return binding


@pytest.mark.parametrize("bits", [3, 4])
def test_decode_32k_sampled(tq, bits):
    dev = torch.device("cuda")
    B, Hkv, T, d, Hq = 32, 8, 32768, 128, 32
    G, qpg = B * Hkv, Hq // Hkv
    print(f"full-size decode 32K b={bits}: generating and quantizing {G * T} keys", flush=True)
    ctx = tq.Context(d, bits, 0)
    K, _ = wl.outlier_keys_torch(B, Hkv, T, d, seed=2, device=dev)
    Kf = K.view(G * T, d)
    cache = tq.tq_quantize(ctx, Kf)
    q = wl.gaussian_torch((B, Hq, d), 7, dev).view(G, qpg, d).contiguous()
    logits = tq.tq_scores(ctx, q, cache, T=T, ldk=T)
    probs = tq.tq_softmax(logits, 1.0 / math.sqrt(d))
    torch.cuda.synchronize()

    rng = np.random.default_rng(99)
    groups = np.sort(rng.choice(G, 6, replace=False))
    toks = np.concatenate([[0, 1, T - 1], rng.choice(T, 509, replace=False)])
    rows = (groups[:, None] * T + toks[None, :]).reshape(-1)
    idx_t = torch.as_tensor(rows, device=dev)
    X = Kf.index_select(0, idx_t).float().cpu().numpy()
    g = {k: v.index_select(0, idx_t).cpu().numpy() for k, v in cache.items()}
    p = O.make_params(d, bits, 0)
    ref = O.quantize(p, X, return_unpacked=True)
    check_quantized(p, g, ref, X)

    same = np.all(g["codes"] == ref["codes"], axis=1) & np.all(g["signs"] == ref["signs"], axis=1)
    assert same.mean() > 0.99
    Q = q.cpu().numpy().astype(np.float64)
    L = logits.cpu().numpy()
    for gi, grp in enumerate(groups):
        sl = slice(gi * len(toks), (gi + 1) * len(toks))
        want = O.scores(p, Q[grp], ref["codes"][sl], ref["signs"][sl], ref["norms"][sl], ref["rnorms"][sl])
        got = L[grp][:, toks]
        keep = same[sl]
        assert_close(got[:, keep], want[:, keep], what=f"logits group {grp}")
    # softmax at full size: properties that hold at any size (values are
    # checked against the oracle on generator inputs in test_gpu_scores)
    P = probs.cpu().numpy()
    assert np.allclose(P.sum(axis=-1), 1.0, atol=1e-3) and (P >= 0).all()
    assert np.array_equal(P.argmax(axis=-1), L.argmax(axis=-1))
