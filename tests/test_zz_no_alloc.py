"""tq_scores_static (scratch memory inside the library, nothing allocated)
against tq_scores (caller workspace), through the C ABI.

Both run the same query-prep and scores kernels, so the logits must agree bit
for bit; two calls in a row (the second smaller) also show that the shared
static buffer holds no state a call depends on.  The oracle checks the first
call's logits on its own records.
"""

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


def _dev(rec):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in rec.items()}


@pytest.mark.parametrize("bits", [3, 4])
def test_static_scratch_matches_workspace_call(tq, bits):
    d = 128
    ctx = tq.Context(d, bits, 0)
    p = O.make_params(d, bits, 0)
    # call 1: 5 groups x 8 heads x 1500 tokens (ldk 1536); call 2: 2 groups x 3 heads x 300 tokens
    for call, (G, qpg, T, ldk, seed) in enumerate([(5, 8, 1500, 1536, 1), (2, 3, 300, 300, 2)]):
        K = wl.gaussian((G * ldk, d), 100 + seed)
        rec = O.quantize(p, K)
        Q = wl.gaussian((G, qpg, d), 200 + seed)
        q = torch.from_numpy(Q).cuda()
        drec = _dev(rec)
        print(f"static scratch b={bits} call {call}: G={G} qpg={qpg} T={T} ldk={ldk}", flush=True)
        got = tq.tq_scores_static(ctx, q, drec, T=T, ldk=ldk)
        want = tq.tq_scores(ctx, q, drec, T=T, ldk=ldk)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"call {call}: static-scratch logits differ from tq_scores"
        if call == 0:
            g = got.cpu().numpy()
            for gi in range(G):
                sl = slice(gi * ldk, gi * ldk + T)
                ref = O.scores(p, Q[gi].astype(np.float64), rec["codes"][sl], rec["signs"][sl],
                               rec["norms"][sl], rec["rnorms"][sl])
                assert_close(g[gi], ref, what=f"logits group {gi}")


def test_static_scratch_limit(tq):
    d = 128
    ctx = tq.Context(d, 3, 0)
    # prepared queries of 1 group x 12000 heads: 3000 head groups x 6400 B > TQ_SCRATCH_BYTES
    G, qpg, T = 1, 12000, 16
    ws = ctx.workspace(tq.TQ_OP_SCORES, G, qpg)
    assert ws.numel() > tq.TQ_SCRATCH_BYTES
    rec = ctx.empty_records(T)
    q = torch.zeros((G, qpg, d), device="cuda")
    logits = torch.full((G, qpg, T), 3.0, device="cuda")
    with pytest.raises(tq.TQError) as e:
        tq.tq_scores_static(ctx, q, rec, T=T, ldk=T, logits=logits)
    assert e.value.status == tq.TQ_ESCRATCH
    torch.cuda.synchronize()
    assert (logits == 3.0).all()
