"""Seeded synthetic inputs shaped like the workloads the TurboQuant pages describe.

This module holds random-number recipes only -- none of the method's
arithmetic -- so that the tests can hand the very same arrays to the GPU path
and to the CPU oracle.  Small inputs come from NumPy's PCG64
(``default_rng(seed)``), large ones from torch's generator on the target
device (same law, not the same bytes).

Recipes (the pages evaluate on models and datasets that are not available
here, so these stand in for them):
  * keys with a few extreme channels (suzuke blog, "技術上怎麼做到的 / 第一步":
    some dimensions are much larger than others): per KV head, 4 channels
    chosen without replacement are scaled by 10; all entries N(0,1) otherwise.
  * anisotropic vectors, covariance eigenvalues 1/i (power-law spectrum,
    exponent 1), axis aligned; optionally normalised to unit length (stand-in
    for GloVe d=200, xujun.org note 189244, "常见问题").
  * random packed records (uniform bytes, positive norms) for estimator tests.
"""

import numpy as np

try:  # torch is plumbing for device memory; the CPU paths do not need it
    import torch
except Exception:  # pragma: no cover
    torch = None


# ----------------------------------------------------------------- NumPy side
def gaussian(shape, seed, dtype=np.float32):
    """iid N(0,1) float64 draws cast to ``dtype``."""
    return np.random.default_rng(seed).standard_normal(shape).astype(dtype)


def tiny_case(seed=0, n=4096, d=128, nq=16):
    """Keys [n, d] then queries [nq, d], fp32 iid N(0,1), keys drawn first."""
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((n, d)).astype(np.float32)
    Q = rng.standard_normal((nq, d)).astype(np.float32)
    return K, Q


def outlier_channels(n_heads, d, seed, n_out=4):
    """Per KV head, ``n_out`` distinct channel ids (drawn first from the seed)."""
    rng = np.random.default_rng(seed)
    return np.stack([rng.choice(d, n_out, replace=False) for _ in range(n_heads)])


def outlier_keys_np(B, H, T, d, seed, scale=10.0):
    """Keys [B, H, T, d] float32 with 4 outlier channels per head (x scale)."""
    rng = np.random.default_rng(seed)
    ch = np.stack([rng.choice(d, 4, replace=False) for _ in range(H)])
    K = rng.standard_normal((B, H, T, d)).astype(np.float32)
    for h in range(H):
        K[:, h, :, ch[h]] *= scale
    return K, ch


def power_law(n, d, seed, exponent=1.0, unit=False):
    """Rows g * sqrt(lambda), lambda_i = i^-exponent (i = 1..d), fp32."""
    rng = np.random.default_rng(seed)
    lam = np.arange(1, d + 1, dtype=np.float64) ** (-exponent)
    X = rng.standard_normal((n, d)) * np.sqrt(lam)[None, :]
    if unit:
        X /= np.linalg.norm(X, axis=1, keepdims=True)
    return X.astype(np.float32)


def random_records(n, code_bytes, sign_bytes, seed):
    """Uniform random code/sign bytes (padding bits included) and positive norms."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, (n, code_bytes), dtype=np.uint8)
    signs = rng.integers(0, 256, (n, sign_bytes), dtype=np.uint8)
    norms = (np.abs(rng.standard_normal(n)) * 8.0 + 0.5).astype(np.float32)
    rnorms = (rng.random(n) * 0.6).astype(np.float32)
    return codes, signs, norms, rnorms


def bf16_round(x):
    """Round float32 to bfloat16 (round-to-nearest-even) and widen back to fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


# ----------------------------------------------------------------- torch side
def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def outlier_keys_torch(B, H, T, d, seed, device, dtype=None, scale=10.0):
    """Device keys [B, H, T, d] (default bf16) with 4 outlier channels per head.

    The outlier channel ids come from :func:`outlier_channels` (NumPy, same
    seed); the bulk is torch.randn on ``device`` with a generator seeded by
    ``seed``.  Generated one head at a time to bound temporary memory.
    """
    dtype = dtype or torch.bfloat16
    ch = outlier_channels(H, d, seed)
    g = _gen(device, seed)
    out = torch.empty((B, H, T, d), dtype=dtype, device=device)
    mult = torch.ones((H, d), dtype=torch.float32, device=device)
    for h in range(H):
        mult[h, torch.as_tensor(ch[h], device=device)] = scale
    for b in range(B):
        for h in range(H):
            x = torch.randn((T, d), generator=g, device=device, dtype=torch.float32)
            out[b, h] = (x * mult[h]).to(dtype)
    return out, ch


def gaussian_torch(shape, seed, device, dtype=torch.float32 if torch else None):
    g = _gen(device, seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(dtype)


def power_law_torch(n, d, seed, device, dtype=None, exponent=1.0, unit=False):
    dtype = dtype or torch.bfloat16
    g = _gen(device, seed)
    lam = torch.arange(1, d + 1, device=device, dtype=torch.float64) ** (-exponent)
    sl = lam.sqrt().to(torch.float32)
    out = torch.empty((n, d), dtype=dtype, device=device)
    step = 1 << 18
    for s in range(0, n, step):
        x = torch.randn((min(step, n - s), d), generator=g, device=device) * sl
        if unit:
            x = x / x.norm(dim=1, keepdim=True)
        out[s:s + step] = x.to(dtype)
    return out
