"""CPU tests of the C-ABI library: exports, host-side parameters, validation.

No compute call is made here (no GPU in this environment): only host logic.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "oblivious_kv_cache_amd", "lib", "libtq.so")
HEADER = os.path.join(ROOT, "include", "tq.h")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libtq.so not built")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert "tq_init" in names and "tq_scores" in names and "tq_topk" in names
    lib = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(lib, n), n
    from oblivious_kv_cache_amd import binding
    assert sorted(binding.EXPORTS) == names


@pytest.mark.parametrize("d,bits,mode,seed", [
    (128, 3, "prod", 0), (128, 2, "prod", 1), (128, 4, "prod", 7), (200, 2, "prod", 0),
    (200, 4, "prod", 0), (64, 3, "mse", 1), (8, 1, "mse", 3), (256, 4, "mse", 5), (96, 3, "prod", 11),
    (520, 3, "prod", 2), (1024, 4, "prod", 4), (1024, 2, "mse", 6),
])
def test_host_params_match_oracle(d, bits, mode, seed):
    from oblivious_kv_cache_amd import binding as tq
    Pi, S, c, t = tq.tq_host_params(d, bits, seed, tq.TQ_MODE_PROD if mode == "prod" else tq.TQ_MODE_MSE)
    p = O.make_params(d, bits, seed, mode)
    assert np.abs(Pi - p.Pi).max() < 1e-12
    assert S.shape == p.S.shape and (S.size == 0 or np.abs(S - p.S).max() < 1e-12)
    assert np.abs(c - p.c).max() < 1e-13 and np.abs(t - p.t).max() < 1e-13
    assert np.array_equal(c, -c[::-1])


def test_host_params_validation():
    from oblivious_kv_cache_amd import binding as tq
    for d, bits, mode in [(7, 3, 0), (0, 3, 0), (1032, 3, 0), (1020, 3, 0), (128, 1, 0), (128, 5, 0), (128, 0, 1),
                          (128, 5, 1), (128, 3, 2)]:
        with pytest.raises(tq.TQError) as e:
            tq.tq_host_params(d, bits, 0, mode)
        assert e.value.status == tq.TQ_EINVAL


def test_argument_validation_before_any_device_work():
    from oblivious_kv_cache_amd import binding as tq
    L = tq.LIB
    h = ctypes.c_void_p()
    assert L.tq_init(7, 3, 0, ctypes.byref(h)) == tq.TQ_EINVAL
    assert L.tq_init(128, 5, 0, ctypes.byref(h)) == tq.TQ_EINVAL
    assert L.tq_init_mse(128, 0, 0, ctypes.byref(h)) == tq.TQ_EINVAL
    assert h.value is None                    # *out untouched on error
    assert L.tq_init(128, 3, 0, None) == tq.TQ_EINVAL
    assert L.tq_quantize(None, None, 0, 1, 128, 1, None, None, None, None, None) == tq.TQ_EINVAL
    assert L.tq_scores(None, None, 1, 4, 1, 1, None, None, None, None, None, None, 0, None) == tq.TQ_EINVAL
    assert L.tq_prep_queries(None, None, 1, 4, None, 0, None) == tq.TQ_EINVAL
    assert L.tq_decode_step(None, None, None, 1, 4, None, None, tq.TQ_F32, 128, 0, 1, None, None, None, None,
                            None, None, 1.0, None, None, None, None, 0, None) == tq.TQ_EINVAL
    assert L.tq_decode_prep(None, None, None, 1, 4, None, None, tq.TQ_F32, 128, 0, 1, None, None, None, None,
                            None, None, None, 0, None) == tq.TQ_EINVAL
    assert L.tq_scores_prepared(None, None, 0, 1, 4, 1, 1, None, None, None, None, None, None) == tq.TQ_EINVAL
    assert L.tq_scores_prepared_timed(None, None, 0, 1, 4, 1, 1, None, None, None, None, None, None,
                                      None, None) == tq.TQ_EINVAL
    assert L.tq_softmax(None, -1, 4, 1.0, None, None) == tq.TQ_EINVAL
    assert L.tq_softmax(None, 0, 4, 1.0, None, None) == tq.TQ_OK          # empty: nothing to do
    assert L.tq_dequant(None, None, None, None, None, 1, None, None) == tq.TQ_EINVAL
    assert L.tq_topk(None, None, 1, 1, None, None, None, None, 1, None, None, None, 0, None) == tq.TQ_EINVAL
    assert L.tq_attend(None, None, None, 1, 4, 1, 1, None, None, None, None, None, None, 1.0,
                       None, None, None, None, 0, None) == tq.TQ_EINVAL
    n = ctypes.c_size_t()
    assert L.tq_workspace_size(None, tq.TQ_OP_SCORES, 1, 4, 0, ctypes.byref(n)) == tq.TQ_EINVAL
    L.tq_free(None)                           # null-safe
    assert tq.tq_strerror(tq.TQ_EINVAL) == "invalid argument"
    assert tq.tq_strerror(12345) == "unknown status"


@pytest.mark.parametrize("d,bits", [(32, 1), (64, 3), (128, 2), (128, 4), (256, 3)])
def test_polar_codebooks_match_oracle(d, bits):
    # the library's own Lloyd-Max iteration for the angle laws (C++, its own
    # Gauss-Legendre rule) against the oracle's
    import oracle.polar as PQ
    from oblivious_kv_cache_amd import binding as tq
    c, t = tq.tq_polar_codebook(d, bits)
    books = PQ.codebooks(d, bits)
    assert c.shape == (len(books), 2 ** bits)
    for level, (bc, bt) in enumerate(books):
        assert np.abs(c[level] - bc).max() < 1e-12 and np.abs(t[level] - bt).max() < 1e-12
    with pytest.raises(tq.TQError):
        tq.tq_polar_codebook(96, bits)          # not a power of two


@pytest.mark.parametrize("d,hb,seed", [(128, 5, 0), (256, 7, 3), (128, 7, 9)])
def test_host_params_fractional_widths_match_oracle(d, hb, seed):
    import oracle.frac as F
    from oblivious_kv_cache_amd import binding as tq
    Pi, S, c, t = tq.tq_host_params(d, hb, seed, tq.TQ_MODE_FRAC)
    p = F.FracParams(d, hb, seed)
    assert np.abs(Pi - p.Pi).max() < 1e-12 and np.abs(S - p.S).max() < 1e-12
    nh = p.c_hi.size
    assert c.size == nh + p.c_lo.size and t.size == c.size - 2
    assert np.abs(c[:nh] - p.c_hi).max() < 1e-13 and np.abs(c[nh:] - p.c_lo).max() < 1e-13
    assert np.abs(t[:nh - 1] - p.t_hi).max() < 1e-13 and np.abs(t[nh - 1:] - p.t_lo).max() < 1e-13
    for d_bad, hb_bad in [(128, 6), (128, 3), (192, 5), (64, 7), (512, 5)]:
        with pytest.raises(tq.TQError):
            tq.tq_host_params(d_bad, hb_bad, 0, tq.TQ_MODE_FRAC)
