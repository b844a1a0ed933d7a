"""GPU parity: PolarQuant contexts (tq_init_polar) -- tq_quantize (the
recursive polar transform of the rotated vector, per-level angle codes) and
tq_dequant (reconstruction from the centroid angles) -- against the oracle
(oracle/polar.py)."""

import numpy as np
import pytest

import oracle.polar as PQ
from oblivious_kv_cache_amd import workloads as wl
from parity import assert_close, check_polar

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from oblivious_kv_cache_amd import binding
    return binding


def _quantize(tq, d, bits, X, dtype, seed=0):
    ctx = tq.Context(d, bits, seed, tq.TQ_MODE_POLAR)
    xt = torch.from_numpy(np.ascontiguousarray(X)).cuda().to(dtype)
    rec = tq.tq_quantize(ctx, xt)
    torch.cuda.synchronize()
    assert rec["signs"] is None and rec["rnorms"] is None
    g = {"codes": rec["codes"].cpu().numpy(), "norms": rec["norms"].cpu().numpy()}
    return ctx, rec, g, xt.float().cpu().numpy()


@pytest.mark.parametrize("d,bits,n,bf16", [
    (128, 3, 1000, True), (128, 4, 777, False), (128, 1, 300, True), (128, 2, 17, False),
    (64, 3, 513, False), (32, 2, 100, True), (32, 4, 65, False), (256, 3, 300, True), (256, 1, 129, False),
])
def test_polar_quantize_matches_oracle(tq, d, bits, n, bf16):
    X = wl.power_law(n, d, seed=d + bits, exponent=1.0)
    X[::37] *= 40.0
    if n > 10:
        X[5] = 0.0                                     # a zero vector
        X[7] *= 1e-39                                  # a vector below the float32 normal range
    if bf16:
        X = wl.bf16_round(X)
    print(f"polar quantize d={d} b={bits} n={n} {'bf16' if bf16 else 'fp32'}", flush=True)
    ctx, _, g, xin = _quantize(tq, d, bits, X, torch.bfloat16 if bf16 else torch.float32)
    p = PQ.PolarParams(d, bits, 0)
    check_polar(p, g, xin)


@pytest.mark.parametrize("d,bits", [(128, 3), (64, 1), (256, 4), (32, 2)])
def test_polar_dequant_matches_oracle(tq, d, bits):
    # the GPU decodes the oracle's own records
    p = PQ.PolarParams(d, bits, 0)
    X = wl.gaussian((257, d), 70 + d)
    X[3] = 0.0
    rec = PQ.quantize(p, X)
    ctx = tq.Context(d, bits, 0, tq.TQ_MODE_POLAR)
    drec = {"codes": torch.from_numpy(rec["codes"]).cuda(), "norms": torch.from_numpy(rec["norms"]).cuda()}
    got = tq.tq_dequant(ctx, drec).cpu().numpy()
    want = PQ.dequant(p, rec["codes"], rec["norms"])
    assert_close(got, want, what="polar reconstruction")


def test_polar_params_and_errors(tq):
    ctx = tq.Context(128, 3, 0, tq.TQ_MODE_POLAR)
    assert ctx.mode == tq.TQ_MODE_POLAR and ctx.code_bytes == 48 and ctx.sign_bytes == 0
    Pi, _, c, t = ctx.params()
    p = PQ.PolarParams(128, 3, 0)
    assert np.abs(Pi - p.Pi).max() < 1e-12
    for level in range(p.L):
        assert np.abs(c[level] - p.books[level][0]).max() < 1e-12
        assert np.abs(t[level] - p.books[level][1]).max() < 1e-12
    for d in (100, 16, 512):
        with pytest.raises(tq.TQError):
            tq.Context(d, 3, 0, tq.TQ_MODE_POLAR)
    # the estimator calls need a prod-mode context
    assert tq.LIB.tq_scores(ctx.handle, None, 1, 4, 8, 8, None, None, None, None, None, None, 0,
                            None) == tq.TQ_EINVAL


def test_polar_quantize_2p20_sampled(tq):
    # the streaming-quantize shape: 2^20 power-law bf16 vectors, d=128, b=3
    n, d, bits = 1 << 20, 128, 3
    print("polar quantize 2^20 x 128 bf16 b=3", flush=True)
    X = wl.power_law_torch(n, d, seed=3, device=torch.device("cuda"))
    ctx = tq.Context(d, bits, 0, tq.TQ_MODE_POLAR)
    rec = tq.tq_quantize(ctx, X)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(9).choice(n, 1500, replace=False))
    idx = torch.as_tensor(rows, device="cuda")
    g = {k: rec[k].index_select(0, idx).cpu().numpy() for k in ("codes", "norms")}
    check_polar(PQ.PolarParams(d, bits, 0), g, X.index_select(0, idx).float().cpu().numpy())
