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

TQ_OK, TQ_EINVAL, TQ_ENOTSUP, TQ_ENOMEM, TQ_EHIP, TQ_ESCRATCH = 0, -1, -2, -3, -4, -5
TQ_SCRATCH_BYTES = 16 << 20
TQ_F32, TQ_BF16 = 0, 1
TQ_MODE_PROD, TQ_MODE_MSE, TQ_MODE_POLAR, TQ_MODE_FRAC = 0, 1, 2, 3
TQ_OP_SCORES, TQ_OP_ATTEND, TQ_OP_TOPK = 1, 2, 3
TQ_MAX_D, TQ_MAX_TOPK = 1024, 1024

EXPORTS = [
    "tq_init", "tq_init_mse", "tq_free", "tq_layout", "tq_host_params", "tq_get_params",
    "tq_quantize", "tq_workspace_size", "tq_scores", "tq_prep_queries", "tq_scores_prepared",
    "tq_scores_prepared_timed",
    "tq_softmax", "tq_attend", "tq_decode_prep", "tq_decode_step", "tq_dequant", "tq_topk",
    "tq_scores_static", "tq_init_polar", "tq_polar_codebook", "tq_init_frac", "tq_strerror",
]


class TQError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: {tq_strerror(status)} ({status})")
        self.status = status


class TQArgError(TQError, ValueError):
    """An argument the binding rejects before calling the library (a buffer
    smaller than the call would touch, a wrong dtype, layout or device):
    status TQ_EINVAL, and nothing is launched or written."""

    def __init__(self, msg):
        RuntimeError.__init__(self, msg)
        self.status = TQ_EINVAL


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
        "tq_init_polar": (I, [I, I, U64, ctypes.POINTER(P)]),
        "tq_init_frac": (I, [I, I, U64, ctypes.POINTER(P)]),
        "tq_polar_codebook": (I, [I, I, D, D]),
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
        "tq_scores_static": (I, [P, P, I64, I, I64, I64, P, P, P, P, P, P]),
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


def _check_tensor(name, t, dtype, min_elems, device=None, check_device=True):
    """Checks one argument tensor before its pointer crosses the C ABI (the
    library cannot see buffer sizes): dtype, contiguity, size and device.
    Sizes are checked before the device, so a wrong shape is reported as
    such wherever the tensor lives."""
    if t is None:
        raise TQArgError(f"{name} is missing")
    if t.dtype != dtype:
        raise TQArgError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise TQArgError(f"{name} must be contiguous")
    if t.numel() < min_elems:
        raise TQArgError(f"{name} holds {t.numel()} elements, the call touches {min_elems}")
    if check_device:
        _check_device(name, t, device)


def _check_device(name, t, device=None):
    if t.device.type != "cuda":
        raise TQArgError(f"{name} must be a device (cuda) tensor, got {t.device}")
    if device is not None and t.device != device:
        raise TQArgError(f"{name} is on {t.device}, expected {device}")


def _check_records(ctx, rec, nrec, what, device=None):
    """The record tensors of ``rec`` must hold at least ``nrec`` records of
    ctx's layout (codes/signs uint8, norms/rnorms float32, contiguous, on
    the device)."""
    if nrec <= 0:
        return
    parts = [("codes", torch.uint8, ctx.code_bytes), ("norms", torch.float32, 1)]
    if ctx.sketch:
        parts += [("signs", torch.uint8, ctx.sign_bytes), ("rnorms", torch.float32, 1)]
    for key, dt, per in parts:
        _check_tensor(f"{what} {key}", rec.get(key), dt, nrec * per, check_device=False)
    for key, _, _ in parts:
        _check_device(f"{what} {key}", rec[key], device)


def _nrec(rec, ctx):
    """Records held by the codes tensor of ``rec``."""
    return rec["codes"].numel() // max(ctx.code_bytes, 1)


def _check_queries(ctx, q, shape, what="q", device=None):
    """Queries: float32, contiguous, the given shape (last dim = ctx.d)."""
    if tuple(q.shape) != tuple(shape):
        raise TQArgError(f"{what} must have shape {tuple(shape)}, got {tuple(q.shape)}")
    _check_tensor(what, q, torch.float32, 0, device)


def _check_rows(ctx, x, n, what):
    """Input vectors: [n, d] fp32 or bf16, unit column stride, row stride a
    multiple of 16 bytes, on the device."""
    if x.dim() != 2 or x.shape[0] != n or x.shape[1] != ctx.d or (n > 0 and x.stride(1) != 1):
        raise TQArgError(f"{what} must be [{n}, {ctx.d}] with unit column stride, got "
                         f"{tuple(x.shape)} strides {tuple(x.stride())}")
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TQArgError(f"{what} must be float32 or bfloat16, got {x.dtype}")
    if x.device.type != "cuda":
        raise TQArgError(f"{what} must be a device (cuda) tensor, got {x.device}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dp(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def tq_host_params(d, bits, seed, mode=TQ_MODE_PROD):
    """Host-only float64 parameters (Pi, S, c, t) a context would hold; needs no GPU."""
    import numpy as np
    if mode == TQ_MODE_FRAC:          # bits = twice the bits per coordinate: both halves' codebooks
        n = 2 ** ((bits + 1) // 2 - 1) + 2 ** (bits // 2 - 1) if bits in (5, 7) else 1
        m = d
    else:
        w = bits - 1 if mode == TQ_MODE_PROD else bits
        n = 2 ** w if 1 <= w <= 4 else 1
        m = d if mode == TQ_MODE_PROD else 0
    Pi = np.zeros((d, d))
    S = np.zeros((max(m, 1), d))
    c = np.zeros(n)
    t = np.zeros(max(n - 1, 1))
    _check(LIB.tq_host_params(d, bits, seed, mode, _dp(Pi), _dp(S), _dp(c), _dp(t)), "tq_host_params")
    return Pi, S[:m], c, t[:n - 2] if mode == TQ_MODE_FRAC else t


def tq_polar_codebook(d, bits):
    """Host-only float64 angle codebooks of a PolarQuant context: (c [L, 2^bits],
    t [L, 2^bits - 1]) for levels 1..L = log2(d)."""
    import numpy as np
    L = max(int(d).bit_length() - 1, 1)
    c = np.zeros((L, 2 ** bits))
    t = np.zeros((L, max(2 ** bits - 1, 1)))
    _check(LIB.tq_polar_codebook(int(d), int(bits), _dp(c), _dp(t)), "tq_polar_codebook")
    return c, t[:, : 2 ** bits - 1]


class Context:
    """Owns a ``tq_ctx *`` (device constants for one (d, bits, seed, mode))."""

    def __init__(self, d, bits, seed=0, mode=TQ_MODE_PROD):
        h = ctypes.c_void_p()
        fn = {TQ_MODE_PROD: LIB.tq_init, TQ_MODE_MSE: LIB.tq_init_mse, TQ_MODE_POLAR: LIB.tq_init_polar,
              TQ_MODE_FRAC: LIB.tq_init_frac}[mode]
        _check(fn(int(d), int(bits), int(seed), ctypes.byref(h)), "tq_init")
        self.handle = h
        lay = tq_layout_t()
        _check(LIB.tq_layout(h, ctypes.byref(lay)), "tq_layout")
        self.layout = lay
        self.d, self.m, self.bits, self.w = lay.d, lay.m, lay.bits, lay.code_bits
        self.code_bytes, self.sign_bytes, self.mode = lay.code_bytes, lay.sign_bytes, lay.mode
        self.seed = seed
        # records with a QJL sketch (signs and residual norms)
        self.sketch = self.mode in (TQ_MODE_PROD, TQ_MODE_FRAC)

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
        if self.mode == TQ_MODE_FRAC:     # both halves' codebooks, first then second
            Pi, S = np.zeros((d, d)), np.zeros((m, d))
            n = L + L // 2
            c, t = np.zeros(n), np.zeros(n - 2)
            _check(LIB.tq_get_params(self.handle, _dp(Pi), _dp(S), _dp(c), _dp(t)), "tq_get_params")
            return Pi, S, (c[:L], c[L:]), (t[:L - 1], t[L - 1:])
        nl = d.bit_length() - 1 if self.mode == TQ_MODE_POLAR else 1   # polar: a codebook per level
        Pi, S = np.zeros((d, d)), np.zeros((max(m, 1), d))
        c, t = np.zeros(nl * L), np.zeros(max(nl * (L - 1), 1))
        _check(LIB.tq_get_params(self.handle, _dp(Pi), _dp(S), _dp(c), _dp(t)), "tq_get_params")
        if self.mode == TQ_MODE_POLAR:
            return Pi, S[:m], c.reshape(nl, L), t[: nl * (L - 1)].reshape(nl, L - 1)
        return Pi, S[:m], c, t[: L - 1]

    def workspace(self, op, a, b, c=0, device="cuda"):
        n = ctypes.c_size_t()
        _check(LIB.tq_workspace_size(self.handle, op, int(a), int(b), int(c), ctypes.byref(n)),
               "tq_workspace_size")
        return torch.empty(max(int(n.value), 16), dtype=torch.uint8, device=device)

    def empty_records(self, n, device="cuda"):
        """Allocate packed-record buffers for n vectors."""
        prod = self.sketch
        return {
            "codes": torch.zeros((n, self.code_bytes), dtype=torch.uint8, device=device),
            "signs": torch.zeros((n, self.sign_bytes), dtype=torch.uint8, device=device) if prod else None,
            "norms": torch.zeros(n, dtype=torch.float32, device=device),
            "rnorms": torch.zeros(n, dtype=torch.float32, device=device) if prod else None,
        }


def tq_quantize(ctx, x, out=None, ldr=1):
    """Quantize rows of x [n, d] (fp32 or bf16, row stride x.stride(0)).

    Vector i goes to record i * ldr of ``out`` (a dict of record tensors whose
    first element is where vector 0 goes).  Without ``out``, buffers of
    (n - 1) * ldr + 1 records are allocated."""
    n = x.shape[0] if x.dim() == 2 else -1
    _check_rows(ctx, x, n, "x")
    ldr = int(ldr)
    if ldr < 1:
        raise TQArgError("ldr must be >= 1")
    dtype = TQ_F32 if x.dtype == torch.float32 else TQ_BF16
    need = (n - 1) * ldr + 1 if n > 0 else 0
    if out is None:
        out = ctx.empty_records(need, x.device)
    _check_records(ctx, out, need, "out", x.device)
    _check(LIB.tq_quantize(ctx.handle, _ptr(x), dtype, n, x.stride(0), ldr, _ptr(out["codes"]),
                           _ptr(out["signs"]), _ptr(out["norms"]), _ptr(out["rnorms"]), _stream()),
           "tq_quantize")
    return out


def _key_span(ctx, rec, G, T, ldk):
    """(ldk, T) defaulted from the record count, and the records a [G][ldk]
    call over T tokens touches: (G - 1) * ldk + T."""
    n = _nrec(rec, ctx)
    ldk = int(ldk) if ldk is not None else n // max(G, 1)
    T = int(T) if T is not None else ldk
    if T < 0 or ldk < T:
        raise TQArgError(f"need 0 <= T <= ldk (T={T}, ldk={ldk})")
    return ldk, T, ((G - 1) * ldk + T if G > 0 and T > 0 else 0)


def _ws_check(ctx, ws, op, a, b, c=0):
    n = ctypes.c_size_t()
    _check(LIB.tq_workspace_size(ctx.handle, op, int(a), int(b), int(c), ctypes.byref(n)), "tq_workspace_size")
    _check_tensor("ws", ws, torch.uint8, int(n.value))


def tq_scores(ctx, q, rec, T=None, ldk=None, logits=None, ws=None):
    """Logits [G, qpg, T] for q [G, qpg, d] against key records laid out [G][ldk]."""
    if q.dim() != 3:
        raise TQArgError("q must be [G, qpg, d]")
    G, qpg, _ = q.shape
    _check_queries(ctx, q, (G, qpg, ctx.d))
    ldk, T, need = _key_span(ctx, rec, G, T, ldk)
    _check_records(ctx, rec, need, "keys", q.device)
    if logits is None:
        logits = torch.empty((G, qpg, T), dtype=torch.float32, device=q.device)
    _check_tensor("logits", logits, torch.float32, G * qpg * T, q.device)
    if ws is None:
        ws = ctx.workspace(TQ_OP_SCORES, G, qpg, device=q.device)
    _ws_check(ctx, ws, TQ_OP_SCORES, G, qpg)
    _check(LIB.tq_scores(ctx.handle, _ptr(q), G, qpg, T, ldk, _ptr(rec["codes"]), _ptr(rec["signs"]),
                         _ptr(rec["norms"]), _ptr(rec["rnorms"]), _ptr(logits), _ptr(ws), ws.numel(),
                         _stream()), "tq_scores")
    return logits


def tq_prep_queries(ctx, q, ws=None):
    """Prepared query state for q [G, qpg, d] (a workspace tensor, returned)."""
    if q.dim() != 3:
        raise TQArgError("q must be [G, qpg, d]")
    G, qpg, _ = q.shape
    _check_queries(ctx, q, (G, qpg, ctx.d))
    if ws is None:
        ws = ctx.workspace(TQ_OP_SCORES, G, qpg, device=q.device)
    _ws_check(ctx, ws, TQ_OP_SCORES, G, qpg)
    _check(LIB.tq_prep_queries(ctx.handle, _ptr(q), G, qpg, _ptr(ws), ws.numel(), _stream()),
           "tq_prep_queries")
    return ws


def tq_scores_prepared(ctx, ws, G, qpg, rec, T=None, ldk=None, logits=None, events=None):
    """Logits [G, qpg, T] from a workspace made by tq_prep_queries.

    events: optional (start, stop) pair of timing-enabled torch.cuda.Event; the
    scores kernel's own dispatch records them (tq_scores_prepared_timed), so
    start.elapsed_time(stop) is that kernel's execution time."""
    G, qpg = int(G), int(qpg)
    ldk, T, need = _key_span(ctx, rec, G, T, ldk)
    _ws_check(ctx, ws, TQ_OP_SCORES, G, qpg)
    _check_records(ctx, rec, need, "keys", ws.device)
    if logits is None:
        logits = torch.empty((G, qpg, T), dtype=torch.float32, device=ws.device)
    _check_tensor("logits", logits, torch.float32, G * qpg * T, ws.device)
    args = (ctx.handle, _ptr(ws), ws.numel(), G, qpg, T, ldk, _ptr(rec["codes"]), _ptr(rec["signs"]),
            _ptr(rec["norms"]), _ptr(rec["rnorms"]), _ptr(logits), _stream())
    if events is None:
        _check(LIB.tq_scores_prepared(*args), "tq_scores_prepared")
    else:
        _check(LIB.tq_scores_prepared_timed(*args, _event_handle(events[0]), _event_handle(events[1])),
               "tq_scores_prepared_timed")
    return logits


def tq_scores_static(ctx, q, rec, T=None, ldk=None, logits=None):
    """tq_scores with the prepared queries in the library's static scratch
    buffer (no workspace, nothing allocated by the library)."""
    if q.dim() != 3:
        raise TQArgError("q must be [G, qpg, d]")
    G, qpg, _ = q.shape
    _check_queries(ctx, q, (G, qpg, ctx.d))
    ldk, T, need = _key_span(ctx, rec, G, T, ldk)
    _check_records(ctx, rec, need, "keys", q.device)
    if logits is None:
        logits = torch.empty((G, qpg, T), dtype=torch.float32, device=q.device)
    _check_tensor("logits", logits, torch.float32, G * qpg * T, q.device)
    _check(LIB.tq_scores_static(ctx.handle, _ptr(q), G, qpg, T, ldk, _ptr(rec["codes"]), _ptr(rec["signs"]),
                                _ptr(rec["norms"]), _ptr(rec["rnorms"]), _ptr(logits), _stream()),
           "tq_scores_static")
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
    T = logits.shape[-1]
    rows = logits.numel() // T if logits.numel() else 0
    _check_tensor("logits", logits, torch.float32, rows * T)
    probs = probs if probs is not None else torch.empty_like(logits)
    _check_tensor("probs", probs, torch.float32, rows * T, logits.device)
    _check(LIB.tq_softmax(_ptr(logits), rows, T, float(scale), _ptr(probs), _stream()), "tq_softmax")
    return probs


def tq_dequant(ctx, rec, out=None):
    n = _nrec(rec, ctx)
    _check_records(ctx, rec, n, "records")
    dev = rec["codes"].device
    out = out if out is not None else torch.empty((n, ctx.d), dtype=torch.float32, device=dev)
    _check_tensor("out", out, torch.float32, n * ctx.d, dev)
    _check(LIB.tq_dequant(ctx.handle, _ptr(rec["codes"]), _ptr(rec.get("signs")), _ptr(rec["norms"]),
                          _ptr(rec.get("rnorms")), n, _ptr(out), _stream()), "tq_dequant")
    return out


def tq_attend(kctx, vctx, q, krec, vrec, scale, T=None, ldk=None, want_logits=False,
              want_probs=False, ws=None):
    if q.dim() != 3:
        raise TQArgError("q must be [G, qpg, d]")
    G, qpg, d = q.shape
    _check_queries(kctx, q, (G, qpg, kctx.d))
    ldk, T, need = _key_span(kctx, krec, G, T, ldk)
    dev = q.device
    _check_records(kctx, krec, need, "keys", dev)
    _check_records(vctx, vrec, need, "values", dev)
    logits = torch.empty((G, qpg, T), dtype=torch.float32, device=dev) if want_logits or want_probs else None
    probs = torch.empty((G, qpg, T), dtype=torch.float32, device=dev) if want_probs else None
    out = torch.empty((G, qpg, d), dtype=torch.float32, device=dev)
    ws = ws if ws is not None else kctx.workspace(TQ_OP_ATTEND, G, qpg, T, device=dev)
    _ws_check(kctx, ws, TQ_OP_ATTEND, G, qpg, T)
    _check(LIB.tq_attend(kctx.handle, vctx.handle, _ptr(q), G, qpg, T, ldk, _ptr(krec["codes"]),
                         _ptr(krec["signs"]), _ptr(krec["norms"]), _ptr(krec["rnorms"]),
                         _ptr(vrec["codes"]), _ptr(vrec["norms"]), float(scale), _ptr(logits),
                         _ptr(probs), _ptr(out), _ptr(ws), ws.numel(), _stream()), "tq_attend")
    return out, (logits if want_logits else None), probs


def _check_new(ctx, x, G, what, like=None):
    _check_rows(ctx, x, G, what)
    if like is not None and (x.dtype != like.dtype or x.stride() != like.stride()):
        raise TQArgError(f"{what} must have the dtype and strides of new_k")


def tq_decode_prep(kctx, q, new_k, krec, pos, ldk=None, vctx=None, new_v=None, vrec=None, ws=None):
    """Append new_k (and new_v) [G, d] at token pos of every group's caches and
    prepare q [G, qpg, d] into a scores workspace (returned)."""
    if q.dim() != 3:
        raise TQArgError("q must be [G, qpg, d]")
    G, qpg, d = q.shape
    _check_queries(kctx, q, (G, qpg, kctx.d))
    _check_new(kctx, new_k, G, "new_k")
    if vctx is not None:
        _check_new(vctx, new_v, G, "new_v", new_k)
    dtype = TQ_F32 if new_k.dtype == torch.float32 else TQ_BF16
    pos = int(pos)
    ldk, _, need = _key_span(kctx, krec, G, pos + 1, ldk)
    _check_records(kctx, krec, need, "keys", q.device)
    if vctx is not None:
        _check_records(vctx, vrec, need, "values", q.device)
    ws = ws if ws is not None else kctx.workspace(TQ_OP_SCORES, G, qpg, device=q.device)
    _ws_check(kctx, ws, TQ_OP_SCORES, G, qpg)
    _check(LIB.tq_decode_prep(kctx.handle, vctx.handle if vctx is not None else None, _ptr(q), G, qpg,
                              _ptr(new_k), _ptr(new_v) if vctx is not None else None, dtype,
                              new_k.stride(0), pos, ldk,
                              _ptr(krec["codes"]), _ptr(krec["signs"]), _ptr(krec["norms"]),
                              _ptr(krec["rnorms"]), _ptr(vrec["codes"]) if vctx is not None else None,
                              _ptr(vrec["norms"]) if vctx is not None else None, _ptr(ws), ws.numel(),
                              _stream()), "tq_decode_prep")
    return ws


def tq_decode_step(kctx, vctx, q, new_k, new_v, krec, vrec, pos, scale, ldk=None,
                   want_logits=False, want_probs=False, ws=None):
    """Append new_k / new_v [G, d] (fp32 or bf16) at token pos of every group's
    caches (records laid out [G][ldk]) and attend over tokens 0..pos."""
    if q.dim() != 3:
        raise TQArgError("q must be [G, qpg, d]")
    G, qpg, d = q.shape
    _check_queries(kctx, q, (G, qpg, kctx.d))
    _check_new(kctx, new_k, G, "new_k")
    _check_new(vctx, new_v, G, "new_v", new_k)
    dtype = TQ_F32 if new_k.dtype == torch.float32 else TQ_BF16
    pos = int(pos)
    T = pos + 1
    ldk, _, need = _key_span(kctx, krec, G, T, ldk)
    dev = q.device
    _check_records(kctx, krec, need, "keys", dev)
    _check_records(vctx, vrec, need, "values", dev)
    logits = torch.empty((G, qpg, T), dtype=torch.float32, device=dev) if want_logits or want_probs else None
    probs = torch.empty((G, qpg, T), dtype=torch.float32, device=dev) if want_probs else None
    out = torch.empty((G, qpg, d), dtype=torch.float32, device=dev)
    ws = ws if ws is not None else kctx.workspace(TQ_OP_ATTEND, G, qpg, T, device=dev)
    _ws_check(kctx, ws, TQ_OP_ATTEND, G, qpg, T)
    _check(LIB.tq_decode_step(kctx.handle, vctx.handle, _ptr(q), G, qpg, _ptr(new_k), _ptr(new_v), dtype,
                              new_k.stride(0), pos, ldk, _ptr(krec["codes"]), _ptr(krec["signs"]),
                              _ptr(krec["norms"]), _ptr(krec["rnorms"]), _ptr(vrec["codes"]),
                              _ptr(vrec["norms"]), float(scale), _ptr(logits), _ptr(probs), _ptr(out),
                              _ptr(ws), ws.numel(), _stream()), "tq_decode_step")
    return out, (logits if want_logits else None), probs


def tq_topk(ctx, q, rec, k, ws=None):
    if q.dim() != 2:
        raise TQArgError("q must be [nq, d]")
    nq = q.shape[0]
    _check_queries(ctx, q, (nq, ctx.d))
    n = _nrec(rec, ctx)
    _check_records(ctx, rec, n, "database", q.device)
    k = int(k)
    ids = torch.empty((nq, k), dtype=torch.int64, device=q.device)
    scores = torch.empty((nq, k), dtype=torch.float32, device=q.device)
    ws = ws if ws is not None else ctx.workspace(TQ_OP_TOPK, nq, n, k, device=q.device)
    _ws_check(ctx, ws, TQ_OP_TOPK, nq, n, k)
    _check(LIB.tq_topk(ctx.handle, _ptr(q), nq, n, _ptr(rec["codes"]), _ptr(rec["signs"]),
                       _ptr(rec["norms"]), _ptr(rec["rnorms"]), k, _ptr(ids), _ptr(scores),
                       _ptr(ws), ws.numel(), _stream()), "tq_topk")
    return ids, scores
