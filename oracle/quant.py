"""fp8 KV pages: E4M3 codes with one float32 scale per (token, KV head) row.
Oracle; test infrastructure only.

The pages name quantization as a technique to pair with DELTA, to save memory on
top of DELTA's savings in attention work (DELTA AI summary page, "Future
Directions"); they fix no format.  Format: OCP 8-bit floating point, E4M3 variant (1 sign bit, 4
exponent bits with bias 7, 3 mantissa bits; no infinities; S.1111.111 is NaN;
largest finite magnitude 448; subnormals M/8 * 2^-6).

Readings (the pages are silent on all of them):
* granularity: one scale per (token, KV head) row of D elements, for K and V
  separately.  A decode step writes one token into a page; a single scale for a
  whole page would have to change, and every earlier token of the page be
  re-encoded, whenever a later token raised the page maximum;
* scale = amax / 448 with amax = max |x| over the row, both in float32, so the
  row's largest magnitude encodes as +-448;
* code = round-to-nearest-even of x / scale (float32 division) to E4M3, after
  clamping to [-448, 448]; the sign of a value that rounds to zero is kept;
* a row whose scale is 0 (all zeros, or amax below 448 * 2^-149) gets scale 0
  and all codes 0;
* the value a code stands for is decode(code) * scale, computed in float64;
  attention then runs on those values exactly as on unquantized K/V.
The float32 steps are the precision the decision is taken in on both sides (an
encoded code is an integer decided by floating point).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code (uint8 array) in float64; NaN for S.1111.111."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = sign * np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


# non-negative finite values, indexed by code 0x00 .. 0x7E (ascending in the code)
_POS = e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(x) -> np.ndarray:
    """Round-to-nearest-even E4M3 code of each finite value with |x| <= 448.

    Nearest representable magnitude by search over the 127 non-negative values;
    a tie goes to the even code (the one whose mantissa ends in 0).  The sign bit
    is the sign of x (so -0.0 and negatives rounding to 0 give 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_encode takes finite values in [-448, 448]")
    a = np.abs(x)
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, len(_POS) - 1)
    lo = np.clip(hi - 1, 0, len(_POS) - 1)
    d_hi = np.abs(_POS[hi] - a)
    d_lo = np.abs(a - _POS[lo])
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    return (pick | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def quantize_rows(x):
    """Encode rows of D values: x [..., D] (values exact in float32, e.g. bfloat16
    values) -> (codes uint8 [..., D], scales float32 [...])."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    xs = (x32 / safe[..., None]).astype(np.float32)
    xs = np.clip(xs, -E4M3_MAX, E4M3_MAX)
    codes = e4m3_encode(xs)
    codes = np.where((scale > 0)[..., None], codes, np.uint8(0)).astype(np.uint8)
    return codes, scale


def dequantize_rows(codes, scales) -> np.ndarray:
    """decode(code) * scale per row, float64."""
    return e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[..., None]


def quantize_dequantize(x) -> np.ndarray:
    """The values an fp8 page holds for the rows x [..., D]."""
    c, s = quantize_rows(x)
    return dequantize_rows(c, s)
