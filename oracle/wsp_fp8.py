"""Plain CPU oracle of the FP8 (OCP E4M3) query/key quantisation used by the
low-precision attention variant.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``.

Format (OCP 8-bit floating point, E4M3 "fn" variant): 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits; normal values (1 + m/8) * 2^(e-7) for
e = 1..15 except the all-ones pattern S.1111.111, which is NaN (no
infinities); subnormals (m/8) * 2^-6 for e = 0; largest finite 448.

Quantisation (a plain reading: the pages only report that low precision
pays off in a neighbouring system): per head, scale = 448 / amax, where
amax is the largest |x| of that head over the tensors quantised together
(video and text rows); the code of x is the E4M3 value nearest to
float32(float32(x) * float32(scale)), ties to even, saturated at +-448.
Scale and product are float32 on both sides, so the quantised codes are
bit-comparable; dequantised x ~= code * amax / 448.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(code) -> np.ndarray:
    """float64 value of E4M3 codes (uint8); NaN for S.1111.111."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return s * v


# every finite non-negative code and its value, for nearest-value search
_POS_CODES = np.arange(0, 0x7F, dtype=np.uint8)          # 0x00 .. 0x7E (0x7F is NaN)
_POS_VALS = e4m3_decode(_POS_CODES)


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code (ties to the even code, i.e. even mantissa), |x|
    saturated at 448, sign bit from x (so -0.0 and negative values that
    round to zero give 0x80).  x must be finite."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    # nearest by exhaustive comparison against the 127 non-negative values
    d = np.abs(a[..., None] - _POS_VALS)
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    # among equally near codes prefer the even one (even mantissa = even code)
    even = (_POS_CODES % 2 == 0)
    pick = np.where(cand & even, 1, 0) + np.where(cand, 1, 0)
    code = _POS_CODES[np.argmax(pick, axis=-1)]
    # the sign bit is kept whatever the magnitude rounds to (E4M3 has a
    # signed zero, 0x80)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def fp8_amax(*tensors) -> np.ndarray:
    """Per-head max |x| over [rows, heads, dim] tensors (all of the same head
    count); tensors without rows add nothing (0 if all are empty)."""
    heads = np.asarray(tensors[0]).shape[1]
    per = [np.abs(np.asarray(t, dtype=np.float64)).max(axis=(0, 2)) for t in tensors if np.asarray(t).shape[0]]
    return np.max(np.stack(per), axis=0) if per else np.zeros(heads)


def fp8_scale(amax) -> np.ndarray:
    """float32 per-head scale 448 / amax (1 where amax is 0)."""
    amax = np.asarray(amax, dtype=np.float32)
    return np.where(amax > 0, np.float32(E4M3_MAX) / np.where(amax > 0, amax, 1), 1).astype(np.float32)


def fp8_quantize(x, amax) -> np.ndarray:
    """E4M3 codes of x [rows, heads, dim] with the per-head scale of amax."""
    x = np.asarray(x, dtype=np.float32)
    prod = x * fp8_scale(amax)[None, :, None]          # float32 product
    return e4m3_encode(prod.astype(np.float64))


def fp8_dequantize(code, amax) -> np.ndarray:
    """float64 values code * amax / 448 (what the low-precision path multiplies)."""
    inv = np.where(np.asarray(amax, np.float64) > 0, np.asarray(amax, np.float64) / E4M3_MAX, 0.0)
    return e4m3_decode(code) * inv[None, :, None]
