"""GPU parity: tq_scores and tq_softmax against the oracle.

The GPU scores the oracle's own packed records (or generator-made random
records), so both sides evaluate the estimator on identical inputs.
"""

import numpy as np
import pytest

import oracle as O
from oblivious_kv_cache_amd import workloads as wl
from parity import ATOL, assert_close

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from oblivious_kv_cache_amd import binding
    return binding


def _dev(rec):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in rec.items()}


def _score(tq, ctx, Q, rec, G, T, ldk):
    q = torch.from_numpy(np.ascontiguousarray(Q, dtype=np.float32)).cuda()
    out = tq.tq_scores(ctx, q, _dev(rec), T=T, ldk=ldk)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _oracle_grouped(p, Q, rec, G, T, ldk):
    out = np.zeros((G, Q.shape[1], T))
    for g in range(G):
        sl = slice(g * ldk, g * ldk + T)
        out[g] = O.scores(p, Q[g].astype(np.float64), rec["codes"][sl], rec["signs"][sl],
                          rec["norms"][sl], rec["rnorms"][sl])
    return out


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_scores_tiny_config_on_oracle_records(tq, bits):
    # 4096 keys, 16 fp32 queries, d=128: G=1, qpg=16 (4 head groups)
    K, Q = wl.tiny_case(seed=0)
    p = O.make_params(128, bits, 0)
    rec = O.quantize(p, K)
    ctx = tq.Context(128, bits, 0)
    print(f"scores tiny b={bits} T=4096 qpg=16", flush=True)
    got = _score(tq, ctx, Q[None], rec, 1, 4096, 4096)
    want = O.scores(p, Q.astype(np.float64), rec["codes"], rec["signs"], rec["norms"], rec["rnorms"])
    assert_close(got[0], want, what="logits")


@pytest.mark.parametrize("d,bits,G,qpg,T,ldk", [
    (128, 3, 3, 4, 1000, 1100), (128, 2, 2, 1, 65, 65), (128, 4, 2, 5, 130, 131),
    (128, 3, 1, 8, 1, 1), (200, 2, 2, 4, 777, 777), (200, 4, 1, 4, 500, 512),
    (64, 3, 4, 4, 300, 300), (96, 4, 2, 3, 257, 260), (256, 3, 1, 2, 129, 129), (40, 2, 1, 4, 63, 63),
    # 3-bit codes at every code-word count per lane group (1 .. 6): merged parity words
    (40, 4, 1, 4, 70, 70), (80, 4, 2, 4, 100, 100), (160, 4, 1, 6, 90, 96), (256, 4, 1, 4, 129, 129),
])
def test_scores_random_records(tq, d, bits, G, qpg, T, ldk):
    ctx = tq.Context(d, bits, 0)
    p = O.make_params(d, bits, 0)
    codes, signs, norms, rnorms = wl.random_records(G * ldk, ctx.code_bytes, ctx.sign_bytes, seed=d + bits)
    rec = {"codes": codes, "signs": signs, "norms": norms, "rnorms": rnorms}
    Q = wl.gaussian((G, qpg, d), 21)
    print(f"scores random d={d} b={bits} G={G} qpg={qpg} T={T} ldk={ldk}", flush=True)
    got = _score(tq, ctx, Q, rec, G, T, ldk)
    assert_close(got, _oracle_grouped(p, Q, rec, G, T, ldk), what="logits")


@pytest.mark.parametrize("d,bits,G,qpg,T,ldk", [
    # many queries per key group (every position of a prefill against one key
    # set): two or four head groups per wave, head-group counts that leave 1,
    # 2 or 3 groups in the last wave (its other slots repeat a group and are
    # not stored), ragged T
    (128, 3, 2, 100, 300, 300), (128, 2, 1, 257, 129, 130), (64, 3, 3, 36, 1000, 1000),
    (128, 4, 1, 12, 64, 64), (128, 3, 1, 1024, 70, 70), (128, 2, 2, 28, 257, 260),
    (64, 3, 1, 40, 190, 190),
    # geometry with more than 12 MFMAs per 16 keys: one head group per wave
    (200, 4, 1, 72, 200, 200),
    # 1024 head groups or more (query prep over many blocks per CU), at
    # b = 2, 3, 4, d = 64 and 128, with a partial last head group
    (128, 3, 2, 2048, 100, 100), (64, 2, 4, 1024, 70, 70), (128, 4, 1, 4096, 40, 40),
    (128, 3, 1, 4099, 33, 33),
    # d > 128: the projection GEMM runs 8-wave blocks (twice the A fragments per wave)
    (200, 2, 1, 4100, 50, 50), (256, 4, 2, 2048, 40, 40), (96, 3, 3, 1366, 30, 31),
])
def test_scores_many_queries_per_group(tq, d, bits, G, qpg, T, ldk):
    ctx = tq.Context(d, bits, 0)
    p = O.make_params(d, bits, 0)
    codes, signs, norms, rnorms = wl.random_records(G * ldk, ctx.code_bytes, ctx.sign_bytes, seed=d + bits + qpg)
    rec = {"codes": codes, "signs": signs, "norms": norms, "rnorms": rnorms}
    Q = wl.gaussian((G, qpg, d), 26)
    print(f"scores many queries d={d} b={bits} G={G} qpg={qpg} T={T} ldk={ldk}", flush=True)
    got = _score(tq, ctx, Q, rec, G, T, ldk)
    assert_close(got, _oracle_grouped(p, Q, rec, G, T, ldk), what="logits")


@pytest.mark.parametrize("d", [128, 200])
def test_scores_many_queries_unaligned_queries(tq, d):
    # queries 4 bytes past a 16-byte boundary: the projection GEMM's query
    # loads take the one-float path (4096 head groups)
    G, qpg, T = 1024, 16, 40
    ctx = tq.Context(d, 3, 0)
    p = O.make_params(d, 3, 0)
    codes, signs, norms, rnorms = wl.random_records(G * T, ctx.code_bytes, ctx.sign_bytes, seed=d)
    rec = {"codes": codes, "signs": signs, "norms": norms, "rnorms": rnorms}
    Q = wl.gaussian((G, qpg, d), 27)
    buf = torch.zeros(G * qpg * d + 1, dtype=torch.float32, device="cuda")
    q = buf[1:].view(G, qpg, d)
    q.copy_(torch.from_numpy(np.ascontiguousarray(Q, dtype=np.float32)))
    assert q.data_ptr() % 16 == 4
    print(f"scores many queries, unaligned q: d={d} G={G} qpg={qpg}", flush=True)
    got = tq.tq_scores(ctx, q, _dev(rec), T=T, ldk=T)
    torch.cuda.synchronize()
    assert_close(got.cpu().numpy(), _oracle_grouped(p, Q, rec, G, T, T), what="logits")


def test_scores_query_count_limits(tq):
    ctx = tq.Context(128, 3, 0)
    rec = ctx.empty_records(5)
    with pytest.raises(tq.TQError) as e:                 # qpg above the library's limit
        ctx.workspace(tq.TQ_OP_SCORES, 1, 65537)
    assert e.value.status == tq.TQ_EINVAL
    # G * ceil(qpg / 4) block rows above the grid's limit: refused before any launch
    q = torch.zeros((5, 65536, 128), device="cuda")
    logits = torch.full((5, 65536, 1), 7.0, device="cuda")
    with pytest.raises(tq.TQError) as e:
        tq.tq_scores(ctx, q, rec, T=1, ldk=1, logits=logits)
    assert e.value.status == tq.TQ_ENOTSUP
    assert (logits == 7.0).all()


def test_scores_zero_norm_keys_and_large_queries(tq):
    d, bits = 128, 3
    ctx = tq.Context(d, bits, 0)
    p = O.make_params(d, bits, 0)
    K = wl.gaussian((300, d), 22, np.float64) * 50.0
    K[::7] = 0.0
    rec = O.quantize(p, K)
    Q = wl.gaussian((1, 4, d), 23) * 30.0
    got = _score(tq, ctx, Q, rec, 1, 300, 300)
    want = _oracle_grouped(p, Q, rec, 1, 300, 300)
    # the logit is linear in the key norm and in the query, so scaling keys by
    # 50 and queries by 30 scales the absolute tolerance (stated for unit-scale
    # inputs) by 1500; the relative part is unchanged
    assert_close(got, want, atol=ATOL * 50.0 * 30.0, what="logits")
    assert (got[0][:, ::7] == 0).all()


def test_scores_deterministic(tq):
    d, bits = 128, 3
    ctx = tq.Context(d, bits, 0)
    codes, signs, norms, rnorms = wl.random_records(4 * 2048, ctx.code_bytes, ctx.sign_bytes, seed=3)
    rec = {"codes": codes, "signs": signs, "norms": norms, "rnorms": rnorms}
    Q = wl.gaussian((4, 4, d), 24)
    a = _score(tq, ctx, Q, rec, 4, 2048, 2048)
    b = _score(tq, ctx, Q, rec, 4, 2048, 2048)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("rows,T,scale", [(5, 1000, 0.125), (3, 33, 1.0), (2, 1, 0.5), (1, 70000, 0.088),
                                         (4, 32768, 0.088), (2, 40000, 0.088), (3, 4096, 0.2)])
def test_softmax_matches_oracle(tq, rows, T, scale):
    L = wl.gaussian((rows, T), 25 + T) * 30.0
    lt = torch.from_numpy(L).cuda()
    print(f"softmax rows={rows} T={T}", flush=True)
    got = tq.tq_softmax(lt, scale).cpu().numpy()
    want = O.softmax(L.astype(np.float64), scale)
    assert_close(got, want, atol=1e-6, rtol=1e-4, what="probs")
    inplace = tq.tq_softmax(lt, scale, probs=lt).cpu().numpy()
    assert np.array_equal(inplace, got)


def test_scores_errors(tq):
    ctx = tq.Context(128, 3, 0)
    mse = tq.Context(128, 3, 1, tq.TQ_MODE_MSE)
    rec = ctx.empty_records(10)
    q = torch.zeros((1, 4, 128), device="cuda")
    with pytest.raises(tq.TQError):
        tq.tq_scores(mse, q, rec, T=10, ldk=10)
    with pytest.raises(tq.TQError):
        tq.tq_scores(ctx, q, rec, T=10, ldk=9)          # ldk < T
    ws = ctx.workspace(tq.TQ_OP_SCORES, 1, 4)
    with pytest.raises(tq.TQError):
        tq.tq_scores(ctx, q, rec, T=10, ldk=10, ws=ws[:16])   # workspace too small


def test_prepared_queries_match_tq_scores_and_oracle(tq):
    # tq_prep_queries + tq_scores_prepared == tq_scores (bit for bit), and one
    # prepared workspace scores two different key sets
    d, bits, G, qpg, T = 128, 3, 3, 6, 700
    ctx = tq.Context(d, bits, 0)
    p = O.make_params(d, bits, 0)
    Q = wl.gaussian((G, qpg, d), 61)
    recs = []
    for seed in (62, 63):
        c, sg, nu, ga = wl.random_records(G * T, ctx.code_bytes, ctx.sign_bytes, seed=seed)
        recs.append({"codes": c, "signs": sg, "norms": nu, "rnorms": ga})
    q = torch.from_numpy(np.ascontiguousarray(Q, dtype=np.float32)).cuda()
    print("scores prepared: G=3 qpg=6 T=700, two key sets", flush=True)
    ws = tq.tq_prep_queries(ctx, q)
    for rec in recs:
        dev = _dev(rec)
        got = tq.tq_scores_prepared(ctx, ws, G, qpg, dev, T=T, ldk=T)
        ref = tq.tq_scores(ctx, q, dev, T=T, ldk=T)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        assert_close(got.cpu().numpy(), _oracle_grouped(p, Q, rec, G, T, T), what="logits")


def test_timed_scores_match_and_time_the_kernel(tq):
    # tq_scores_prepared_timed: same logits as tq_scores_prepared; the events
    # recorded by the kernel's dispatch give a positive duration, and events
    # passed to a call that launches nothing (T = 0) keep their earlier times
    d, bits, G, qpg, T = 128, 3, 4, 4, 5000
    ctx = tq.Context(d, bits, 0)
    Q = wl.gaussian((G, qpg, d), 71)
    c, sg, nu, ga = wl.random_records(G * T, ctx.code_bytes, ctx.sign_bytes, seed=72)
    dev = _dev({"codes": c, "signs": sg, "norms": nu, "rnorms": ga})
    q = torch.from_numpy(np.ascontiguousarray(Q, dtype=np.float32)).cuda()
    print("scores timed: G=4 qpg=4 T=5000", flush=True)
    ws = tq.tq_prep_queries(ctx, q)
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    ref = tq.tq_scores_prepared(ctx, ws, G, qpg, dev, T=T, ldk=T)
    for _ in range(3):
        got = tq.tq_scores_prepared(ctx, ws, G, qpg, dev, T=T, ldk=T, events=ev)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        ms = ev[0].elapsed_time(ev[1])
        assert 0.0 < ms < 100.0
    # logits at a base that is 4-byte but not 16-byte aligned: per-float stores
    flat = torch.empty(G * qpg * T + 1, dtype=torch.float32, device="cuda")
    shifted = flat[1:].view(G, qpg, T)
    tq.tq_scores_prepared(ctx, ws, G, qpg, dev, T=T, ldk=T, logits=shifted)
    torch.cuda.synchronize()
    assert torch.equal(shifted, ref)
    empty = torch.empty((G, qpg, 0), dtype=torch.float32, device="cuda")
    tq.tq_scores_prepared(ctx, ws, G, qpg, dev, T=0, ldk=T, logits=empty, events=ev)
    torch.cuda.synchronize()
    assert ev[0].elapsed_time(ev[1]) == ms
