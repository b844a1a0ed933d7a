"""Thin ctypes binding of ``libtq.so`` (same names as the C ABI in ``include/tq.h``).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  torch tensors provide device memory and the current stream.  If the
library is missing, importing this module raises -- there is no fallback.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# TQ_LIBRARY may point at another build of the same library
LIB_PATH = os.environ.get("TQ_LIBRARY") or os.path.join(_HERE, "lib", "libtq.so")

TQ_OK, TQ_EINVAL, TQ_ENOTSUP, TQ_ENOMEM, TQ_EHIP = 0, -1, -2, -3, -4
TQ_F32, TQ_BF16 = 0, 1
TQ_MODE_PROD, TQ_MODE_MSE = 0, 1
TQ_OP_SCORES, TQ_OP_ATTEND, TQ_OP_TOPK = 1, 2, 3
TQ_MAX_D, TQ_MAX_TOPK = 256, 64

EXPORTS = [
    "tq_init", "tq_init_mse", "tq_free", "tq_layout", "tq_host_params", "tq_get_params",
    "tq_quantize", "tq_workspace_size", "tq_scores", "tq_prep_queries", "tq_scores_prepared",
    "tq_scores_prepared_timed",
    "tq_softmax", "tq_attend", "tq_decode_prep", "tq_decode_step", "tq_dequant", "tq_topk",
    "tq_strerror",
]


class TQError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: {tq_strerror(status)} ({status})")
        self.status = status


class tq_layout_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in
                ("d", "m", "bits", "code_bits", "levels", "code_bytes", "sign_bytes", "mode")]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "or python -m oblivious_kv_cache_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, U64, SZ, F = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64,
                            ctypes.c_size_t, ctypes.c_float)
    D = ctypes.POINTER(ctypes.c_double)
    sig = {
        "tq_init": (I, [I, I, U64, ctypes.POINTER(P)]),
        "tq_init_mse": (I, [I, I, U64, ctypes.POINTER(P)]),
        "tq_free": (None, [P]),
        "tq_layout": (I, [P, ctypes.POINTER(tq_layout_t)]),
        "tq_host_params": (I, [I, I, U64, I, D, D, D, D]),
        "tq_get_params": (I, [P, D, D, D, D]),
        "tq_quantize": (I, [P, P, I, I64, I64, I64, P, P, P, P, P]),
        "tq_workspace_size": (I, [P, I, I64, I64, I64, ctypes.POINTER(SZ)]),
        "tq_scores": (I, [P, P, I64, I, I64, I64, P, P, P, P, P, P, SZ, P]),
        "tq_prep_queries": (I, [P, P, I64, I, P, SZ, P]),
        "tq_scores_prepared": (I, [P, P, SZ, I64, I, I64, I64, P, P, P, P, P, P]),
        "tq_scores_prepared_timed": (I, [P, P, SZ, I64, I, I64, I64, P, P, P, P, P, P, P, P]),
        "tq_softmax": (I, [P, I64, I64, F, P, P]),
        "tq_attend": (I, [P, P, P, I64, I, I64, I64, P, P, P, P, P, P, F, P, P, P, P, SZ, P]),
        "tq_decode_prep": (I, [P, P, P, I64, I, P, P, I, I64, I64, I64, P, P, P, P, P, P, P, SZ, P]),
        "tq_decode_step": (I, [P, P, P, I64, I, P, P, I, I64, I64, I64, P, P, P, P, P, P, F, P, P, P, P,
                               SZ, P]),
        "tq_dequant": (I, [P, P, P, P, P, I64, P, P]),
        "tq_topk": (I, [P, P, I64, I64, P, P, P, P, I, P, P, P, SZ, P]),
        "tq_strerror": (ctypes.c_char_p, [I]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()


def tq_strerror(status):
    return LIB.tq_strerror(int(status)).decode()


def _check(status, what):
    if status != TQ_OK:
        raise TQError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dp(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def tq_host_params(d, bits, seed, mode=TQ_MODE_PROD):
    """Host-only float64 parameters (Pi, S, c, t) a context would hold; needs no GPU."""
    import numpy as np
    w = bits - 1 if mode == TQ_MODE_PROD else bits
    m = d if mode == TQ_MODE_PROD else 0
    Pi = np.zeros((d, d))
    S = np.zeros((max(m, 1), d))
    c = np.zeros(2 ** w) if 1 <= w <= 4 else np.zeros(1)
    t = np.zeros(max(2 ** w - 1, 1))
    _check(LIB.tq_host_params(d, bits, seed, mode, _dp(Pi), _dp(S), _dp(c), _dp(t)), "tq_host_params")
    return Pi, S[:m], c, t


class Context:
    """Owns a ``tq_ctx *`` (device constants for one (d, bits, seed, mode))."""

    def __init__(self, d, bits, seed=0, mode=TQ_MODE_PROD):
        h = ctypes.c_void_p()
        fn = LIB.tq_init if mode == TQ_MODE_PROD else LIB.tq_init_mse
        _check(fn(int(d), int(bits), int(seed), ctypes.byref(h)), "tq_init")
        self.handle = h
        lay = tq_layout_t()
        _check(LIB.tq_layout(h, ctypes.byref(lay)), "tq_layout")
        self.layout = lay
        self.d, self.m, self.bits, self.w = lay.d, lay.m, lay.bits, lay.code_bits
        self.code_bytes, self.sign_bytes, self.mode = lay.code_bytes, lay.sign_bytes, lay.mode
        self.seed = seed

    def close(self):
        if getattr(self, "handle", None):
            LIB.tq_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def params(self):
        import numpy as np
        d, m, L = self.d, self.m, 2 ** self.w
        Pi, S, c, t = np.zeros((d, d)), np.zeros((max(m, 1), d)), np.zeros(L), np.zeros(L - 1)
        _check(LIB.tq_get_params(self.handle, _dp(Pi), _dp(S), _dp(c), _dp(t)), "tq_get_params")
        return Pi, S[:m], c, t

    def workspace(self, op, a, b, c=0, device="cuda"):
        n = ctypes.c_size_t()
        _check(LIB.tq_workspace_size(self.handle, op, int(a), int(b), int(c), ctypes.byref(n)),
               "tq_workspace_size")
        return torch.empty(max(int(n.value), 16), dtype=torch.uint8, device=device)

    def empty_records(self, n, device="cuda"):
        """Allocate packed-record buffers for n vectors."""
        prod = self.mode == TQ_MODE_PROD
        return {
            "codes": torch.zeros((n, self.code_bytes), dtype=torch.uint8, device=device),
            "signs": torch.zeros((n, self.sign_bytes), dtype=torch.uint8, device=device) if prod else None,
            "norms": torch.zeros(n, dtype=torch.float32, device=device),
            "rnorms": torch.zeros(n, dtype=torch.float32, device=device) if prod else None,
        }


def tq_quantize(ctx, x, out=None, ldr=1):
    """Quantize rows of x [n, d] (fp32 or bf16, row stride x.stride(0)).

    Vector i goes to record i * ldr of ``out`` (a dict of record tensors whose
    first element is where vector 0 goes)."""
    if x.dim() != 2 or x.stride(1) != 1 or x.shape[1] != ctx.d:
        raise ValueError(f"x must be [n, {ctx.d}] with unit column stride")
    dtype = {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16}[x.dtype]
    n = x.shape[0]
    out = out or ctx.empty_records(n, x.device)
    _check(LIB.tq_quantize(ctx.handle, _ptr(x), dtype, n, x.stride(0), int(ldr), _ptr(out["codes"]),
                           _ptr(out["signs"]), _ptr(out["norms"]), _ptr(out["rnorms"]), _stream()),
           "tq_quantize")
    return out


def tq_scores(ctx, q, rec, T=None, ldk=None, logits=None, ws=None):
    """Logits [G, qpg, T] for q [G, qpg, d] against key records laid out [G][ldk]."""
    G, qpg, d = q.shape
    assert q.is_contiguous() and q.dtype == torch.float32 and d == ctx.d
    n = rec["codes"].shape[0]
    ldk = ldk if ldk is not None else n // max(G, 1)
    T = T if T is not None else ldk
    if logits is None:
        logits = torch.empty((G, qpg, T), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = ctx.workspace(TQ_OP_SCORES, G, qpg, device=q.device)
    _check(LIB.tq_scores(ctx.handle, _ptr(q), G, qpg, T, ldk, _ptr(rec["codes"]), _ptr(rec["signs"]),
                         _ptr(rec["norms"]), _ptr(rec["rnorms"]), _ptr(logits), _ptr(ws), ws.numel(),
                         _stream()), "tq_scores")
    return logits


def tq_prep_queries(ctx, q, ws=None):
    """Prepared query state for q [G, qpg, d] (a workspace tensor, returned)."""
    G, qpg, d = q.shape
    assert q.is_contiguous() and q.dtype == torch.float32 and d == ctx.d
    if ws is None:
        ws = ctx.workspace(TQ_OP_SCORES, G, qpg, device=q.device)
    _check(LIB.tq_prep_queries(ctx.handle, _ptr(q), G, qpg, _ptr(ws), ws.numel(), _stream()),
           "tq_prep_queries")
    return ws


def tq_scores_prepared(ctx, ws, G, qpg, rec, T=None, ldk=None, logits=None, events=None):
    """Logits [G, qpg, T] from a workspace made by tq_prep_queries.

    events: optional (start, stop) pair of timing-enabled torch.cuda.Event; the
    scores kernel's own dispatch records them (tq_scores_prepared_timed), so
    start.elapsed_time(stop) is that kernel's execution time."""
    n = rec["codes"].shape[0]
    ldk = ldk if ldk is not None else n // max(G, 1)
    T = T if T is not None else ldk
    if logits is None:
        logits = torch.empty((G, qpg, T), dtype=torch.float32, device=ws.device)
    args = (ctx.handle, _ptr(ws), ws.numel(), G, qpg, T, ldk, _ptr(rec["codes"]), _ptr(rec["signs"]),
            _ptr(rec["norms"]), _ptr(rec["rnorms"]), _ptr(logits), _stream())
    if events is None:
        _check(LIB.tq_scores_prepared(*args), "tq_scores_prepared")
    else:
        _check(LIB.tq_scores_prepared_timed(*args, _event_handle(events[0]), _event_handle(events[1])),
               "tq_scores_prepared_timed")
    return logits


def _event_handle(ev):
    """The hipEvent_t of a timing-enabled torch.cuda.Event (None -> NULL).  torch
    creates the underlying event at its first record(), so an event that was
    never recorded is recorded once here, on the current stream."""
    if ev is None:
        return None
    if not ev.cuda_event:
        ev.record()
    return ctypes.c_void_p(ev.cuda_event)


def tq_softmax(logits, scale, probs=None):
    rows = logits.numel() // logits.shape[-1] if logits.numel() else 0
    T = logits.shape[-1]
    assert logits.is_contiguous() and logits.dtype == torch.float32
    probs = probs if probs is not None else torch.empty_like(logits)
    _check(LIB.tq_softmax(_ptr(logits), rows, T, float(scale), _ptr(probs), _stream()), "tq_softmax")
    return probs


def tq_dequant(ctx, rec, out=None):
    n = rec["codes"].shape[0]
    out = out if out is not None else torch.empty((n, ctx.d), dtype=torch.float32,
                                                  device=rec["codes"].device)
    _check(LIB.tq_dequant(ctx.handle, _ptr(rec["codes"]), _ptr(rec.get("signs")), _ptr(rec["norms"]),
                          _ptr(rec.get("rnorms")), n, _ptr(out), _stream()), "tq_dequant")
    return out


def tq_attend(kctx, vctx, q, krec, vrec, scale, T=None, ldk=None, want_logits=False,
              want_probs=False, ws=None):
    G, qpg, d = q.shape
    n = krec["codes"].shape[0]
    ldk = ldk if ldk is not None else n // max(G, 1)
    T = T if T is not None else ldk
    dev = q.device
    logits = torch.empty((G, qpg, T), dtype=torch.float32, device=dev) if want_logits else None
    probs = torch.empty((G, qpg, T), dtype=torch.float32, device=dev) if want_probs else None
    out = torch.empty((G, qpg, d), dtype=torch.float32, device=dev)
    ws = ws if ws is not None else kctx.workspace(TQ_OP_ATTEND, G, qpg, T, device=dev)
    _check(LIB.tq_attend(kctx.handle, vctx.handle, _ptr(q), G, qpg, T, ldk, _ptr(krec["codes"]),
                         _ptr(krec["signs"]), _ptr(krec["norms"]), _ptr(krec["rnorms"]),
                         _ptr(vrec["codes"]), _ptr(vrec["norms"]), float(scale), _ptr(logits),
                         _ptr(probs), _ptr(out), _ptr(ws), ws.numel(), _stream()), "tq_attend")
    return out, logits, probs


def tq_decode_prep(kctx, q, new_k, krec, pos, ldk=None, vctx=None, new_v=None, vrec=None, ws=None):
    """Append new_k (and new_v) [G, d] at token pos of every group's caches and
    prepare q [G, qpg, d] into a scores workspace (returned)."""
    G, qpg, d = q.shape
    assert new_k.shape == (G, d) and new_k.stride(1) == 1
    if vctx is not None:
        assert new_v.shape == (G, d) and new_v.dtype == new_k.dtype and new_v.stride() == new_k.stride()
    dtype = {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16}[new_k.dtype]
    n = krec["codes"].shape[0]
    ldk = ldk if ldk is not None else n // max(G, 1)
    ws = ws if ws is not None else kctx.workspace(TQ_OP_SCORES, G, qpg, device=q.device)
    _check(LIB.tq_decode_prep(kctx.handle, vctx.handle if vctx is not None else None, _ptr(q), G, qpg,
                              _ptr(new_k), _ptr(new_v), dtype, new_k.stride(0), int(pos), ldk,
                              _ptr(krec["codes"]), _ptr(krec["signs"]), _ptr(krec["norms"]),
                              _ptr(krec["rnorms"]), _ptr(vrec["codes"]) if vrec is not None else None,
                              _ptr(vrec["norms"]) if vrec is not None else None, _ptr(ws), ws.numel(),
                              _stream()), "tq_decode_prep")
    return ws


def tq_decode_step(kctx, vctx, q, new_k, new_v, krec, vrec, pos, scale, ldk=None,
                   want_logits=False, want_probs=False, ws=None):
    """Append new_k / new_v [G, d] (fp32 or bf16) at token pos of every group's
    caches (records laid out [G][ldk]) and attend over tokens 0..pos."""
    G, qpg, d = q.shape
    assert new_k.shape == (G, d) and new_v.shape == (G, d) and new_k.dtype == new_v.dtype
    assert new_k.stride() == new_v.stride() and new_k.stride(1) == 1
    dtype = {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16}[new_k.dtype]
    n = krec["codes"].shape[0]
    ldk = ldk if ldk is not None else n // max(G, 1)
    T = pos + 1
    dev = q.device
    logits = torch.empty((G, qpg, T), dtype=torch.float32, device=dev) if want_logits else None
    probs = torch.empty((G, qpg, T), dtype=torch.float32, device=dev) if want_probs else None
    out = torch.empty((G, qpg, d), dtype=torch.float32, device=dev)
    ws = ws if ws is not None else kctx.workspace(TQ_OP_ATTEND, G, qpg, T, device=dev)
    _check(LIB.tq_decode_step(kctx.handle, vctx.handle, _ptr(q), G, qpg, _ptr(new_k), _ptr(new_v), dtype,
                              new_k.stride(0), int(pos), ldk, _ptr(krec["codes"]), _ptr(krec["signs"]),
                              _ptr(krec["norms"]), _ptr(krec["rnorms"]), _ptr(vrec["codes"]),
                              _ptr(vrec["norms"]), float(scale), _ptr(logits), _ptr(probs), _ptr(out),
                              _ptr(ws), ws.numel(), _stream()), "tq_decode_step")
    return out, logits, probs


def tq_topk(ctx, q, rec, k, ws=None):
    nq = q.shape[0]
    n = rec["codes"].shape[0]
    ids = torch.empty((nq, k), dtype=torch.int64, device=q.device)
    scores = torch.empty((nq, k), dtype=torch.float32, device=q.device)
    ws = ws if ws is not None else ctx.workspace(TQ_OP_TOPK, nq, n, k, device=q.device)
    _check(LIB.tq_topk(ctx.handle, _ptr(q), nq, n, _ptr(rec["codes"]), _ptr(rec["signs"]),
                       _ptr(rec["norms"]), _ptr(rec["rnorms"]), int(k), _ptr(ids), _ptr(scores),
                       _ptr(ws), ws.numel(), _stream()), "tq_topk")
    return ids, scores
