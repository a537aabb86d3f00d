"""Independent numpy restatements used to pin the oracle.

Nothing here is shared with the oracle or with the HIP path: the number
formats are rebuilt from their bit-field definitions (OCP fp8 e4m3fn, OCP
fp4 e2m1, bfloat16 = upper half of binary32) and rounding is done by a
nearest-value search over the enumerated grid, not by bit manipulation.  The
compressor steps are written in a different but equivalent form (sigmoid
pooling, complex-number RoPE) so that a slip in the oracle's algebra shows.
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------- formats
def e4m3_table() -> np.ndarray:
    """value of every fp8 e4m3fn code 0..255 (NaN for 0x7F / 0xFF)."""
    v = np.empty(256)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 0xF, c & 7
        if e == 0xF and m == 7:
            v[c] = np.nan
            continue
        mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        v[c] = -mag if s else mag
    return v


def e2m1_table() -> np.ndarray:
    """value of every fp4 e2m1 code 0..15."""
    v = np.empty(16)
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        mag = (m / 2.0) * 1.0 if e == 0 else (1 + m / 2.0) * 2.0 ** (e - 1)
        v[c] = -mag if s else mag
    return v


def bf16_value(b) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def nearest_code(values: np.ndarray, table: np.ndarray, codes_pos: np.ndarray,
                 sign_bit: int) -> np.ndarray:
    """Nearest representable value by search, ties to the code whose lowest
    bit is 0 (the even mantissa); magnitudes beyond the largest grid value
    take the largest (the caller decides whether that is allowed).  Negative
    inputs (and -0.0) get ``sign_bit`` or'ed in."""
    vals = np.asarray(values, np.float64)
    mag = np.abs(vals)
    g = table[codes_pos]
    order = np.argsort(g)
    g, cp = g[order], codes_pos[order]
    hi = np.clip(np.searchsorted(g, mag, side="left"), 0, len(g) - 1)
    lo = np.clip(hi - 1, 0, len(g) - 1)
    dlo = np.abs(mag - g[lo])
    dhi = np.abs(g[hi] - mag)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((cp[hi] & 1) == 0) & (hi != lo))
    code = np.where(pick_hi, cp[hi], cp[lo]).astype(np.int64)
    neg = np.signbit(vals)
    return (code | np.where(neg, sign_bit, 0)).astype(np.uint8)


def e4m3_nearest(values) -> np.ndarray:
    t = e4m3_table()
    return nearest_code(values, t, np.arange(0, 0x7F), 0x80)


def e2m1_nearest(values) -> np.ndarray:
    t = e2m1_table()
    return nearest_code(values, t, np.arange(0, 8), 0x8)


def all_bf16() -> np.ndarray:
    """every finite bf16 bit pattern."""
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    e = (b >> 7) & 0xFF
    return b[e != 0xFF]


def closed_form_ue8m0(amax_f32: np.ndarray) -> np.ndarray:
    """The exponent formula the pages print for the fp8 row quantizer:
    max((bits >> 23) - 8 + (mantissa > 0x600000), 114), bits of fp32 amax."""
    bits = np.asarray(amax_f32, np.float32).view(np.uint32)
    e = (bits >> 23).view(np.int32)              # exponent field, below 2^9
    e -= 8
    e += (bits & 0x7FFFFF) > 0x600000
    return np.maximum(e, 114, out=e)


# ---------------------------------------------------------------- compressor
def pool_norm_rope(k0, s0, k1, s1, w, eps, cs):
    """fp64 reference of one compressed row written another way.

    k0,s0 may be None (ratio 1).  Pooling as k1 + sigmoid(s0 - s1)(k0 - k1);
    RMSNorm through numpy's mean; RoPE as the complex product
    (y_even + i y_odd) * (cos + i sin) on the last 64 dims.
    Returns (y, z) in fp64."""
    k1 = bf16_value(k1)
    if k0 is None:
        v = k1
    else:
        k0, s0, s1 = bf16_value(k0), bf16_value(s0), bf16_value(s1)
        sig = 1.0 / (1.0 + np.exp(-(s0 - s1)))
        v = k1 + sig * (k0 - k1)
    y = v / np.sqrt(np.mean(v * v) + eps) * bf16_value(w)
    z = y.copy()
    rot = cs[0::2].astype(np.float64) + 1j * cs[1::2].astype(np.float64)
    c = (y[448::2] + 1j * y[449::2]) * rot
    z[448::2], z[449::2] = c.real, c.imag
    return y, z


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """spacing of bf16 values at |x| (normal range)."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def bf16_nearest(values) -> np.ndarray:
    """bf16 bit patterns nearest to fp64 ``values`` by search over every
    finite bf16 magnitude, ties to the even pattern; magnitudes past the
    largest finite value by half its spacing or more become infinity."""
    vals = np.asarray(values, np.float64)
    pos = np.arange(0, 0x7F81, dtype=np.uint16)              # +0 .. +inf
    g = bf16_value(pos)
    g[-1] = 2.0 ** 128                                       # where infinity begins
    mag = np.abs(vals)
    hi = np.clip(np.searchsorted(g, mag, side="left"), 0, len(g) - 1)
    lo = np.clip(hi - 1, 0, len(g) - 1)
    dlo, dhi = np.abs(mag - g[lo]), np.abs(g[hi] - mag)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((pos[hi] & 1) == 0) & (hi != lo))
    code = np.where(pick_hi, pos[hi], pos[lo]).astype(np.uint16)
    return code | np.where(np.signbit(vals), np.uint16(0x8000), np.uint16(0))
