"""FP8 E4M3 KV-cache values (oracle).

The pages treat a low-precision KV cache as a dequantising key/value
transform with a scale contract (pinghaoyang page, the table of
customisable hooks in "可定制注意力模板：把变化留给 JIT": KeyTransform and
ValueTransform cover dequantisation; section "适用边界与工程取舍": low-precision
KV comes with a scale contract), cite E4M3 KV caches in the vLLM integration
(section "反例比最好数字更能说明集成成本"), and describe quantising new rows
while appending them (pyshine, "The Paged KV Cache Layer").

Readings taken where the pages are silent:
* the format is OCP FP8 E4M3 ("e4m3fn"): sign bit, 4 exponent bits with
  bias 7, 3 mantissa bits, subnormals, no infinities, S.1111.111 is NaN, so
  the largest finite magnitude is 448;
* one float scale per tensor: a stored code c stands for e4m3(c) * scale, and
  a value x is stored as e4m3 of x / scale, rounded to nearest (ties to
  even) and saturated to +-448 (a cache entry must not become NaN).
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_to_f64(bits) -> np.ndarray:
    """Exact value of each E4M3 code (uint8) as float64 (NaN for S.1111.111)."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = m * 2.0 ** -9
    val = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & ((b & 7) == 7), np.nan, val)


def f64_to_e4m3(x) -> np.ndarray:
    """Nearest E4M3 code (ties to even mantissa), saturated to +-448; NaN maps
    to the positive NaN code 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.uint8)
    codes = np.arange(256, dtype=np.uint8)
    vals = e4m3_to_f64(codes)
    finite = ~np.isnan(vals)
    pos = codes[finite & (vals >= 0) & ~((codes >> 7).astype(bool))]  # +0 .. 448
    pos_vals = vals[pos]                                             # increasing
    flat_x = x.reshape(-1)
    flat_o = out.reshape(-1)
    for n, v in enumerate(flat_x):
        if np.isnan(v):
            flat_o[n] = 0x7F
            continue
        a = min(abs(v), E4M3_MAX)
        j = int(np.searchsorted(pos_vals, a))  # pos_vals[j-1] < a <= pos_vals[j]
        if j < len(pos_vals) and pos_vals[j] == a:
            c = int(pos[j])
        else:
            lo, hi = int(pos[j - 1]), int(pos[j])
            dl, dh = a - pos_vals[j - 1], pos_vals[j] - a
            c = lo if dl < dh else hi if dh < dl else (lo if lo % 2 == 0 else hi)
        if v < 0 or (v == 0 and np.signbit(v)):
            c |= 0x80
        flat_o[n] = c
    return out
