"""Counter-based random numbers shared by the host side (oracle, tests) and the
device fill kernels (``workload/csrc/fill.hip``).

Generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers:
as easy as 1, 2, 3", SC'11): a 4x32-bit counter, a 2x32-bit key, ten rounds of
two 32x32->64 multiplies with Weyl key bumps.  Both sides implement it from that
definition; ``tests/test_workload.py`` checks it against the authors' published
known-answer vectors.

Normal variates: each Philox block (4 words) gives four N(0,1) values by the
Box-Muller transform in float64, two per word pair (x_a, x_b):
    u1 = (x_a + 1) * 2^-32   in (0, 1]
    u2 =  x_b      * 2^-32   in [0, 1)
    z  = sqrt(-2 ln u1) * (cos(2 pi u2), sin(2 pi u2))
Element ``e`` of a stream is word pair ``(e % 4) // 2`` of block ``e // 4``,
cosine branch for even ``e``, sine branch for odd ``e``.

Stream addressing: counter = (block, row, layer, kind), key = (seed lo, seed hi).
This module holds no arithmetic of the attention method; it only draws numbers.
"""
from __future__ import annotations

import numpy as np

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
TWO_PI = 6.283185307179586  # nearest double to 2*pi; the device uses the same literal
TWO_M32 = 2.3283064365386963e-10  # 2^-32, exact

# Stream kinds (counter word 3).
KIND_K = 1      # key noise, row = b*Hkv + g, element = t*D + d
KIND_V = 2      # value noise, same addressing as K
KIND_Q = 3      # query noise, row = b*Hq + h, element = step*D + d
KIND_DIR = 4    # salient direction, row = b*Hkv + g, element = d
KIND_POS = 5    # salient / drift positions (raw words), layer word = epoch
KIND_LEN = 6    # ragged prefill lengths (raw words), row = 0

_MASK = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32-10 on broadcastable uint32-valued arrays; returns 4 uint32 arrays."""
    c0 = np.asarray(c0, dtype=np.uint64)
    c1 = np.asarray(c1, dtype=np.uint64)
    c2 = np.asarray(c2, dtype=np.uint64)
    c3 = np.asarray(c3, dtype=np.uint64)
    k0 = np.uint64(int(k0) & 0xFFFFFFFF)
    k1 = np.uint64(int(k1) & 0xFFFFFFFF)
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    s32 = np.uint64(32)
    for rnd in range(10):
        p0 = c0 * m0
        p1 = c2 * m1
        c0, c1, c2, c3 = ((p1 >> s32) ^ c1 ^ k0, p1 & _MASK, (p0 >> s32) ^ c3 ^ k1, p0 & _MASK)
        if rnd != 9:
            k0 = (k0 + np.uint64(PHILOX_W0)) & _MASK
            k1 = (k1 + np.uint64(PHILOX_W1)) & _MASK
    return (c0.astype(np.uint32), c1.astype(np.uint32), c2.astype(np.uint32), c3.astype(np.uint32))


def raw_words(seed: int, kind: int, layer: int, row: int, n_blocks: int, block0: int = 0):
    """Blocks ``block0 .. block0+n_blocks-1`` of one stream as an [n, 4] uint32 array."""
    j = np.arange(block0, block0 + n_blocks, dtype=np.uint64)
    w = philox4x32_10(j, np.uint64(row), np.uint64(layer), np.uint64(kind), seed & 0xFFFFFFFF, seed >> 32)
    return np.stack(w, axis=-1)


def normals(seed: int, kind: int, layer: int, rows, start: int, count: int) -> np.ndarray:
    """float64 N(0,1) elements ``start .. start+count-1`` of streams ``rows``.

    ``rows`` is an int or a 1-D array; the result has shape [len(rows), count]
    (or [count] for an int row).
    """
    scalar = np.isscalar(rows)
    rows_a = np.atleast_1d(np.asarray(rows, dtype=np.uint64))
    if count <= 0:
        out = np.zeros((rows_a.size, 0))
        return out[0] if scalar else out
    b0 = start // 4
    b1 = (start + count - 1) // 4 + 1
    j = np.arange(b0, b1, dtype=np.uint64)[None, :]
    r = rows_a[:, None]
    x0, x1, x2, x3 = philox4x32_10(j, r, np.uint64(layer), np.uint64(kind), seed & 0xFFFFFFFF, seed >> 32)
    z = np.empty((rows_a.size, b1 - b0, 4), dtype=np.float64)
    for (xa, xb, ia) in ((x0, x1, 0), (x2, x3, 2)):
        u1 = (xa.astype(np.float64) + 1.0) * TWO_M32
        u2 = xb.astype(np.float64) * TWO_M32
        rad = np.sqrt(-2.0 * np.log(u1))
        th = TWO_PI * u2
        z[:, :, ia] = rad * np.cos(th)
        z[:, :, ia + 1] = rad * np.sin(th)
    z = z.reshape(rows_a.size, -1)[:, start - 4 * b0: start - 4 * b0 + count]
    return z[0] if scalar else z


def f32_round(x) -> np.ndarray:
    """Round float64 to the nearest float32 (ties to even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def bf16_round(x32) -> np.ndarray:
    """Round float32 to the nearest bfloat16 (ties to even); returned as float32 values."""
    b = np.ascontiguousarray(np.asarray(x32, dtype=np.float32)).view(np.uint32)
    r = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    hi = ((b + r) >> np.uint32(16)).astype(np.uint32)
    return (hi << np.uint32(16)).view(np.float32)


def bf16_bits(x32) -> np.ndarray:
    """uint16 bit patterns of ``bf16_round(x32)``."""
    return (bf16_round(x32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def to_dtype_values(x64, dtype: str) -> np.ndarray:
    """float64 -> the stored element value (float32 or bfloat16), returned as float32."""
    x32 = f32_round(x64)
    return bf16_round(x32) if dtype == "bf16" else x32
