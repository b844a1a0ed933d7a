"""CPU tests of the binding's argument checks (no GPU, no library call).

The C ABI cannot see buffer sizes, so the binding checks every record,
query, output and workspace tensor against what the call would touch before
any pointer crosses it: a wrong size, dtype or layout is a TQArgError
(status TQ_EINVAL, also a ValueError), never an out-of-bounds device access.
Sizes are checked before the device, so these checks run on CPU tensors.
"""

import os
from types import SimpleNamespace

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "oblivious_kv_cache_amd", "lib", "libtq.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libtq.so not built")

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def tq():
    from oblivious_kv_cache_amd import binding
    return binding


def _ctx(tq, d=128, code_bytes=32, sign_bytes=16, prod=True):
    return SimpleNamespace(d=d, code_bytes=code_bytes, sign_bytes=sign_bytes,
                           mode=tq.TQ_MODE_PROD if prod else tq.TQ_MODE_MSE, sketch=prod, handle=None)


def _rec(n, cb=32, sb=16):
    return {"codes": torch.zeros((n, cb), dtype=torch.uint8), "signs": torch.zeros((n, sb), dtype=torch.uint8),
            "norms": torch.zeros(n), "rnorms": torch.zeros(n)}


def test_record_sizes(tq):
    ctx = _ctx(tq)
    # 3 groups x ldk 100, T = 90: the call touches (3 - 1) * 100 + 90 = 290 records
    ldk, T, need = tq._key_span(ctx, _rec(290), 3, 90, 100)
    assert (ldk, T, need) == (100, 90, 290)
    with pytest.raises(tq.TQArgError, match="device"):      # right sizes: only the device is wrong
        tq._check_records(ctx, _rec(290), need, "keys")
    for short in ("codes", "signs", "norms", "rnorms"):
        rec = _rec(290)
        rec[short] = rec[short][:-1]
        with pytest.raises(tq.TQArgError, match=short):
            tq._check_records(ctx, rec, need, "keys")
    with pytest.raises(ValueError):                         # TQArgError is also a ValueError
        tq._check_records(ctx, _rec(289), need, "keys")
    # MSE records need no signs / rnorms
    mse = _ctx(tq, code_bytes=48, sign_bytes=0, prod=False)
    rec = {"codes": torch.zeros((10, 48), dtype=torch.uint8), "norms": torch.zeros(10), "signs": None}
    with pytest.raises(tq.TQArgError, match="device"):
        tq._check_records(mse, rec, 10, "values")


def test_dtypes_layout_and_spans(tq):
    ctx = _ctx(tq)
    rec = _rec(64)
    rec["norms"] = torch.zeros(64, dtype=torch.float64)
    with pytest.raises(tq.TQArgError, match="float32"):
        tq._check_records(ctx, rec, 64, "keys")
    rec = _rec(64)
    rec["codes"] = torch.zeros((32, 64), dtype=torch.uint8).t()     # non-contiguous view
    with pytest.raises(tq.TQArgError, match="contiguous"):
        tq._check_records(ctx, rec, 64, "keys")
    with pytest.raises(tq.TQArgError, match="T <= ldk"):
        tq._key_span(ctx, _rec(64), 1, 65, 64)
    # queries: shape, dtype
    with pytest.raises(tq.TQArgError, match="shape"):
        tq._check_queries(ctx, torch.zeros((2, 4, 127)), (2, 4, 128))
    with pytest.raises(tq.TQArgError, match="float32"):
        tq._check_queries(ctx, torch.zeros((2, 4, 128), dtype=torch.bfloat16), (2, 4, 128))
    # input rows of quantize
    with pytest.raises(tq.TQArgError, match="unit column stride"):
        tq._check_rows(ctx, torch.zeros((128, 4)).t(), 4, "x")
    with pytest.raises(tq.TQArgError, match="float32 or bfloat16"):
        tq._check_rows(ctx, torch.zeros((4, 128), dtype=torch.float16), 4, "x")


def test_quantize_checks_record_span_with_stride(tq):
    # ldr = 3, n = 5: vector 4 goes to record 12, so 13 records are touched
    ctx = _ctx(tq)
    x = torch.zeros((5, 128))
    with pytest.raises(tq.TQArgError, match="device"):
        tq.tq_quantize(ctx, x, out=_rec(13), ldr=3)
    with pytest.raises(tq.TQArgError):
        tq.tq_quantize(ctx, x, out=_rec(12), ldr=3)
