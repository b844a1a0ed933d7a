"""Quantize / pack / dequantize (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Steps, in the pages' order:
 1. keep the vector's length (xujun.org note 189244, "第一步：PolarQuant": a
    final radius survives; nothing else per block is stored);
 2. rotate the unit vector by Pi (suzuke blog, "第一步");
 3. per-coordinate Max-Lloyd code (suzuke blog, "第二步"): index = number of
    thresholds strictly below the coordinate (a tie on a threshold takes the
    lower index);
 4. residual of stage 1 and its length (xujun.org note 189244, "第二步：QJL");
 5. JL projection of that residual, one sign bit per row (xujun.org note
    189244, "第二步：QJL"; suzuke blog, "第三步"); sign(0) counts as +1.

Packed record layout (the pages fix none; this is the library's layout):
  codes[n][code_bytes]: prod mode (keys): little-endian bit stream, code i in
  bits [i*w, (i+1)*w), LSB first; MSE-only mode (values): w bit planes of d
  bits each, plane p in bytes [p d/8, (p+1) d/8) holding bit p of code i at
  bit i of the plane (d is a multiple of 8); signs[n][sign_bytes]: bit j =
  (byte j>>3, bit j&7), 1 <=> +1; norms[n], rnorms[n] float32.  Record byte
  counts are rounded up to a multiple of 16 and the padding is zero.  A zero
  vector encodes as all-zero codes and signs with norm 0 and residual norm 0.
"""

import numpy as np


def _round16(x):
    return (x + 15) // 16 * 16


def record_sizes(d, w, m):
    """(code_bytes, sign_bytes) of one packed record."""
    cb = _round16((d * w + 7) // 8)
    sb = _round16((m + 7) // 8) if m else 0
    return cb, sb


def pack_bits(values, width, nbytes):
    """Pack rows of small unsigned ints ``values[n, k]`` at ``width`` bits each."""
    values = np.asarray(values, dtype=np.uint64)
    n, k = values.shape
    bits = ((values[:, :, None] >> np.arange(width, dtype=np.uint64)) & np.uint64(1)).astype(np.uint8)
    bits = bits.reshape(n, k * width)
    out = np.zeros((n, nbytes * 8), dtype=np.uint8)
    out[:, : k * width] = bits
    return np.packbits(out, axis=1, bitorder="little")


def unpack_bits(packed, width, k):
    """Inverse of :func:`pack_bits`: ``k`` values of ``width`` bits per row."""
    packed = np.asarray(packed, dtype=np.uint8)
    bits = np.unpackbits(packed, axis=1, bitorder="little")[:, : k * width]
    bits = bits.reshape(packed.shape[0], k, width).astype(np.int64)
    return (bits << np.arange(width, dtype=np.int64)).sum(axis=2)


def pack_planes(values, width, d, nbytes):
    """Bit planes of rows ``values[n, d]``: plane p (bit p of every value) as d
    bits, value i at bit i, planes one after another; ``nbytes`` per row."""
    values = np.asarray(values, dtype=np.int64)
    n = values.shape[0]
    out = np.zeros((n, nbytes * 8), dtype=np.uint8)
    for plane in range(width):
        out[:, plane * d:(plane + 1) * d] = (values >> plane) & 1
    return np.packbits(out, axis=1, bitorder="little")


def unpack_planes(packed, width, d):
    """Inverse of :func:`pack_planes`: [n, d] values of ``width`` bits."""
    bits = np.unpackbits(np.asarray(packed, dtype=np.uint8), axis=1, bitorder="little").astype(np.int64)
    out = np.zeros((bits.shape[0], d), dtype=np.int64)
    for plane in range(width):
        out |= bits[:, plane * d:(plane + 1) * d] << plane
    return out


def pack_codes(p, idx):
    """Code records of a context: bit stream (prod) or bit planes (MSE-only)."""
    cb = record_sizes(p.d, p.w, p.m)[0]
    if p.mode == "mse":
        return pack_planes(idx, p.w, p.d, cb)
    return pack_bits(idx, p.w, cb)


def unpack_codes(p, codes):
    """Code indices [n, d] from a context's code records."""
    if p.mode == "mse":
        return unpack_planes(codes, p.w, p.d)
    return unpack_bits(codes, p.w, p.d)


def quantize_one(p, x):
    """Quantize one vector ``x[d]`` step by step.

    Returns (idx[d] int, sign_bits[m] int, norm float32, rnorm float32).
    """
    x = np.asarray(x, dtype=np.float64)
    nu = float(np.sqrt(np.sum(x * x)))
    if nu == 0.0:
        return (np.zeros(p.d, np.int64), np.zeros(p.m, np.int64),
                np.float32(0.0), np.float32(0.0))
    u = x / nu
    y = p.Pi @ u
    idx = np.array([int(np.sum(p.t < yi)) for yi in y], dtype=np.int64)
    if p.mode == "mse":
        return idx, np.zeros(0, np.int64), np.float32(nu), np.float32(0.0)
    r = y - p.c[idx]
    gamma = float(np.sqrt(np.sum(r * r)))
    resid_orig = u - p.Pi.T @ p.c[idx]          # stage-1 error in x's coordinates
    z = p.S @ resid_orig
    bits = (z >= 0.0).astype(np.int64)
    return idx, bits, np.float32(nu), np.float32(gamma)


def stage2_from_codes(p, x, idx):
    """Residual norm and sign bits of one vector for a given stage-1 code choice.

    Used where two stage-1 codes are both valid (a coordinate on a threshold
    within rounding): the QJL stage is then evaluated for the given codes.
    Returns (gamma float64, z [m] float64, bits [m] int).
    """
    x = np.asarray(x, np.float64)
    nu = float(np.sqrt(np.sum(x * x)))
    u = x / nu
    y = p.Pi @ u
    r = y - p.c[np.asarray(idx)]
    gamma = float(np.sqrt(np.sum(r * r)))
    z = p.S @ (u - p.Pi.T @ p.c[np.asarray(idx)])
    return gamma, z, (z >= 0.0).astype(np.int64)


def quantize(p, X, chunk=65536, return_unpacked=False):
    """Batched form of :func:`quantize_one` (same arithmetic, BLAS GEMMs).

    ``X`` is [n, d] (any float dtype; widened exactly to float64).
    Returns dict(codes, signs, norms, rnorms) in the packed layout, plus
    ``idx``, ``sbits``, ``y``, ``z`` (float64 intermediates) if asked.
    """
    X = np.asarray(X)
    n = X.shape[0]
    cb, sb = record_sizes(p.d, p.w, p.m)
    codes = np.zeros((n, cb), np.uint8)
    signs = np.zeros((n, sb), np.uint8)
    norms = np.zeros(n, np.float32)
    rnorms = np.zeros(n, np.float32)
    extra = {"idx": [], "sbits": [], "y": [], "z": []}
    for s in range(0, n, chunk):
        x = X[s:s + chunk].astype(np.float64)
        nu = np.sqrt(np.sum(x * x, axis=1))
        zero = nu == 0.0
        u = x / np.where(zero, 1.0, nu)[:, None]
        y = u @ p.Pi.T
        idx = np.searchsorted(p.t, y, side="left")   # = #{k : t_k < y}
        idx[zero] = 0
        codes[s:s + chunk] = pack_codes(p, idx)
        norms[s:s + chunk] = nu.astype(np.float32)
        if p.mode == "prod":
            r = y - p.c[idx]
            gamma = np.sqrt(np.sum(r * r, axis=1))
            gamma[zero] = 0.0
            z = (u - p.c[idx] @ p.Pi) @ p.S.T
            bits = (z >= 0.0).astype(np.int64)
            bits[zero] = 0
            signs[s:s + chunk] = pack_bits(bits, 1, sb)
            rnorms[s:s + chunk] = gamma.astype(np.float32)
        else:
            z, bits = np.zeros((len(x), 0)), np.zeros((len(x), 0), np.int64)
        if return_unpacked:
            extra["idx"].append(idx)
            extra["sbits"].append(bits)
            extra["y"].append(np.where(zero[:, None], 0.0, y))
            extra["z"].append(z)
    out = {"codes": codes, "signs": signs, "norms": norms, "rnorms": rnorms}
    if return_unpacked:
        for k, v in extra.items():
            out[k] = np.concatenate(v) if v else np.zeros((0,))
    return out


def dequant(p, codes, signs, norms, rnorms):
    """Reconstruct x_hat [n, d] from packed records.

    prod: x_hat = nu (Pi^T c[idx] + alpha gamma S^T (2 bits - 1));
    mse:  x_hat = nu Pi^T c[idx]
    (suzuke blog, "第三步": approximation plus residual correction).
    """
    idx = unpack_codes(p, codes)
    nu = np.asarray(norms, np.float64)[:, None]
    xhat = p.c[idx] @ p.Pi
    if p.mode == "prod":
        sb = unpack_bits(signs, 1, p.m).astype(np.float64)
        gamma = np.asarray(rnorms, np.float64)[:, None]
        xhat = xhat + p.alpha * gamma * ((2.0 * sb - 1.0) @ p.S)
    return nu * xhat
