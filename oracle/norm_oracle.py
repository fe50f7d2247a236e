"""fp64 CPU oracle of the gated RMSNorm + FP8 quantisation that follows the GDN
recurrence.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it follows
---------------
"The inference stack behind OCRia" (LlamaIndex), section on avoiding needless
memory traffic by fusing kernels: the GDN output goes through a gated RMSNorm
that is followed by FP8 quantisation, done in one kernel so the normalised
values never make a round trip to HBM. The pages give no formula; the reading
taken (listed in the design notes) is the usual gated RMSNorm of GDN layers,
per (token, value head), over the d_v outputs o of that head:

    r   = sqrt(mean_j o_j^2 + eps)
    y_j = (o_j / r) * w_j * silu(z_j),      silu(x) = x / (1 + exp(-x))

with a weight w shared by the heads and a gate z (the output-gate projection,
bf16). FP8 is OCP E4M3 (the "fn" variant: bias 7, 3 mantissa bits, no
infinities, largest finite 448, code 0x7F / 0xFF is NaN), one scale per
(token, head) group of d_v values:

    s   = max_j |y_j| / 448      (1 when every y_j is 0)
    c_j = E4M3(y_j / s)          round to nearest, ties to even, saturating

so the group dequantises as c_j * s.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_BIAS = 7


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    """OCP E4M3 code (uint8) -> float64 value (NaN for 0x7F / 0xFF)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = sign * (1.0 + m / 8.0) * np.exp2(e - E4M3_BIAS)
    sub = sign * (m / 8.0) * np.exp2(1 - E4M3_BIAS)
    v = np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


# every finite non-negative value in code order (codes 0x00 .. 0x7E)
_POS = e4m3_decode(np.arange(0x7F))


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float64 -> OCP E4M3 code: round to nearest, ties to the even code (the
    one whose mantissa LSB is 0), saturating at +-448; -0.0 and values that
    round to zero keep their sign bit."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    # index of the largest representable value <= a
    lo = np.searchsorted(_POS, a, side="right") - 1
    hi = np.minimum(lo + 1, 0x7E)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    up = (d_hi < d_lo) | ((d_hi == d_lo) & (hi != lo) & ((lo & 1) == 1))
    code = np.where(up, hi, lo).astype(np.int64)
    sign = np.signbit(x)
    return (code | np.where(sign, 0x80, 0)).astype(np.uint8)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def gated_rmsnorm(o: np.ndarray, z: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """y over the last axis (d_v) of o [..., d_v] (fp64)."""
    o = np.asarray(o, dtype=np.float64)
    r = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return (o / r) * np.asarray(weight, dtype=np.float64) * silu(np.asarray(z, dtype=np.float64))


def group_scale(y: np.ndarray) -> np.ndarray:
    """s = max |y| / 448 over the last axis, 1 for an all-zero group."""
    amax = np.max(np.abs(y), axis=-1)
    return np.where(amax > 0, amax / E4M3_MAX, 1.0)


def gated_rmsnorm_fp8(o, z, weight, eps):
    """(y, s, c): the fp64 normalised values, the per-group scales and the codes
    of y / s."""
    y = gated_rmsnorm(o, z, weight, eps)
    s = group_scale(y)
    return y, s, e4m3_encode(y / s[..., None])
