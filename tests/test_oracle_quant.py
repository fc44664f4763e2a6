"""Pins for oracle.quant (fp8 E4M3 KV rows with per-row scales).

Library routine: torch's float8_e4m3fn dtype (OCP E4M3) for decoding every code
and for round-to-nearest-even encoding, ties included.  Closed forms: the format's
landmark values, the exact round trip of representable rows, the relative error
bound of a 3-bit mantissa."""
import numpy as np
import pytest
import torch

from oracle import quant as Q


def test_decode_matches_torch_float8_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = Q.e4m3_decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    fin = ~np.isnan(ref)
    assert np.array_equal(ref[fin], got[fin])
    assert np.array_equal(np.signbit(ref[fin]), np.signbit(got[fin]))


def test_decode_landmarks():
    v = Q.e4m3_decode(np.array([0x38, 0x7E, 0x08, 0x07, 0x01, 0x00, 0x80, 0x7F, 0xFF, 0xFE, 0x40], dtype=np.uint8))
    assert v[0] == 1.0 and v[1] == 448.0 and v[2] == 2.0 ** -6      # one, largest, smallest normal
    assert v[3] == 7 / 8 * 2.0 ** -6 and v[4] == 2.0 ** -9          # largest / smallest subnormal
    assert v[5] == 0.0 and v[6] == 0.0 and np.signbit(v[6])
    assert np.isnan(v[7]) and np.isnan(v[8]) and v[9] == -448.0 and v[10] == 2.0
    assert np.sum(np.isfinite(Q.e4m3_decode(np.arange(256, dtype=np.uint8)))) == 254


def _midpoints():
    p = Q.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    return (p[1:] + p[:-1]) / 2


def test_encode_matches_torch_rne_including_ties():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(100_000) * 40, rng.standard_normal(20_000) * 1e-2,
                        _midpoints(), -_midpoints(), [0.0, -0.0, 1e-30, -1e-30, 448.0, -448.0, 447.9]])
    x = np.clip(x, -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(Q.e4m3_encode(x), ref)


def test_encode_roundtrip_and_range():
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(Q.e4m3_encode(Q.e4m3_decode(finite)), finite)
    with pytest.raises(ValueError):
        Q.e4m3_encode(np.array([449.0]))


def test_quantize_rows_exact_on_representable_rows():
    """A row that is 2^k times E4M3 values with largest magnitude 448 has scale 2^k
    exactly and round-trips without error."""
    rng = np.random.default_rng(9)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    rows = Q.e4m3_decode(rng.choice(finite, size=(50, 128)))
    rows[:, 7] = 448.0 * np.where(rng.random(50) < 0.5, 1, -1)
    rows *= np.exp2(rng.integers(-20, 4, size=50))[:, None]
    codes, scales = Q.quantize_rows(rows)
    assert np.array_equal(scales.astype(np.float64), np.abs(rows).max(axis=1) / 448.0)
    assert np.array_equal(Q.dequantize_rows(codes, scales), rows)


def test_quantize_rows_error_bound_and_landmarks():
    rng = np.random.default_rng(11)
    x = torch.from_numpy(rng.standard_normal((64, 128)) * 3).to(torch.bfloat16).double().numpy()
    codes, scales = Q.quantize_rows(x)
    assert scales.dtype == np.float32
    assert np.array_equal(scales, (np.abs(x).max(axis=1).astype(np.float32) / np.float32(448)).astype(np.float32))
    # the row maximum encodes as +-448
    imax = np.abs(x).argmax(axis=1)
    assert np.all((codes[np.arange(64), imax] & 0x7F) == 0x7E)
    dq = Q.dequantize_rows(codes, scales)
    xs = np.abs(x) / scales[:, None].astype(np.float64)
    normal = xs >= 2.0 ** -6
    # 3 mantissa bits: half an ulp is 2^-4 of the binade's lower end
    assert np.all(np.abs(dq - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal] * (1 + 1e-6))
    assert np.all(np.abs(dq - x)[~normal] <= 2.0 ** -10 * np.broadcast_to(scales[:, None], x.shape)[~normal] * (1 + 1e-6))
    assert np.array_equal(np.sign(dq[dq != 0]), np.sign(x[dq != 0]))


def test_zero_row():
    codes, scales = Q.quantize_rows(np.zeros((3, 64)))
    assert np.all(codes == 0) and np.all(scales == 0)
    assert np.all(Q.dequantize_rows(codes, scales) == 0)
