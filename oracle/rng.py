"""Counter-based random numbers for the method's own random draws (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The method draws a random orthogonal matrix and a Gaussian JL matrix from a
seed (suzuke blog, "技術上怎麼做到的 / 第一步": multiply by a random
orthogonal matrix; xujun.org note 189244, "第二步：QJL": Johnson-Lindenstrauss
projection).  The pages do not name a generator, so both this oracle and the
library implement, independently, SplitMix64 as published by Steele, Lea and
Flood ("Fast splittable pseudorandom number generators", OOPSLA 2014), in its
counter form, followed by the Box-Muller transform (Box and Muller, 1958).

Definition used here (written from those publications):
  gamma      = 0x9E3779B97F4A7C15
  state0     = seed XOR ((stream + 1) * gamma)            (mod 2^64)
  out[i]     = mix64(state0 + (i + 1) * gamma)            (mod 2^64)
  mix64(z)   : z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9
               z = (z ^ (z >> 27)) * 0x94D049BB133111EB
               return z ^ (z >> 31)
  normal k   : u1 = ((out[2k] >> 11) + 1) * 2^-53   in (0, 1]
               u2 = (out[2k+1] >> 11) * 2^-53       in [0, 1)
               g  = sqrt(-2 ln u1) * cos(2 pi u2)
"""

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def _mix64(z):
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64_stream(seed, stream, count):
    """Return ``count`` uint64 SplitMix64 outputs of sub-stream ``stream``."""
    with np.errstate(over="ignore"):
        state0 = np.uint64(seed) ^ (np.uint64(stream + 1) * GAMMA)
        i = np.arange(1, count + 1, dtype=np.uint64)
        return _mix64(state0 + i * GAMMA)


def gaussian_stream(seed, stream, count):
    """Return ``count`` float64 N(0,1) draws (Box-Muller, cosine branch only)."""
    raw = splitmix64_stream(seed, stream, 2 * count)
    u1 = ((raw[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0**-53
    u2 = (raw[1::2] >> np.uint64(11)).astype(np.float64) * 2.0**-53
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
