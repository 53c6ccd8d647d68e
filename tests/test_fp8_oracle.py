"""Pins of the FP8 (E4M3) cache oracle (oracle/fp8_cache.py), CPU only.

The format is pinned against torch's own float8_e4m3fn type (an independent
implementation of the same OCP E4M3 format) and against hand-derived values; the
quantizer against its defining properties (the row maximum lands on 448, the error
bound of one rounding, zero rows)."""
import numpy as np
import pytest
import torch

import oracle.fp8_cache as f8

ALL = np.arange(256, dtype=np.uint8)


def test_hand_values():
    v = f8.e4m3_value(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x3C, 0x40, 0x7E, 0x7F, 0x80, 0xB8,
                                0xFE, 0xFF], np.uint8))
    assert v[0] == 0.0
    assert v[1] == 2.0 ** -9                  # smallest subnormal: 1/8 * 2^-6
    assert v[2] == 7 * 2.0 ** -9              # largest subnormal
    assert v[3] == 2.0 ** -6                  # smallest normal
    assert v[4] == 1.0 and v[5] == 1.5 and v[6] == 2.0
    assert v[7] == 448.0                      # largest finite: 1.75 * 2^8
    assert np.isnan(v[8]) and np.isnan(v[12])
    assert v[9] == 0.0 and np.signbit(v[9])   # 0x80 is -0
    assert v[10] == -1.0 and v[11] == -448.0


def test_decode_matches_torch_float8_e4m3fn():
    ref = torch.from_numpy(ALL.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = f8.e4m3_value(ALL)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])


def test_round_trip_of_every_finite_code():
    fin = ~np.isnan(f8.e4m3_value(ALL))
    assert np.array_equal(f8.e4m3_round(f8.e4m3_value(ALL[fin])), ALL[fin])


def test_rounding_matches_torch_on_random_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 40, rng.uniform(-448, 448, 20000),
                        rng.standard_normal(5000) * 2.0 ** -8]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(f8.e4m3_round(x), ref)


def test_ties_go_to_the_even_code():
    vals = f8.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2          # every midpoint between neighbours
    codes = f8.e4m3_round(mids)
    assert np.all(codes % 2 == 0)
    assert np.all((codes == np.arange(0x7E)) | (codes == np.arange(1, 0x7F)))
    # by hand: 1.0625 lies between 1.0 (0x38) and 1.125 (0x39) -> 1.0; 1.1875 between
    # 1.125 (0x39) and 1.25 (0x3A) -> 1.25; 2^-10 between 0 and 2^-9 -> 0
    assert list(f8.e4m3_round([1.0625, 1.1875, 2.0 ** -10, -1.1875])) == [0x38, 0x3A, 0x00, 0xBA]
    # torch agrees on the midpoints
    ref = torch.from_numpy(mids.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


def test_saturation_nan_and_signed_zero():
    assert list(f8.e4m3_round([448.0, 460.0, 1e6, -500.0, np.inf])) == [0x7E, 0x7E, 0x7E, 0xFE, 0x7E]
    assert f8.e4m3_round([np.nan])[0] == 0x7F
    assert list(f8.e4m3_round([-0.0, 0.0, -1e-30])) == [0x80, 0x00, 0x80]


def test_scale_exponent_by_hand():
    # smallest e with amax <= 448 * 2^e: 448 -> 0, 448.0001 -> 1, 224 -> -1, 224.5 -> 0,
    # 1 -> -8 (448 / 256 = 1.75 >= 1), 1.75 -> -8, 1.76 -> -7; clamps at -124 and 117
    amax = [448.0, 448.0001, 224.0, 224.5, 1.0, 1.75, 1.76, 2.0 ** -130, 2.0 ** 127, 0.0]
    assert list(f8.scale_exponent(amax)) == [0, 1, -1, 0, -8, -8, -7, -124, 117, 0]


def test_quantized_row_maximum_lands_in_224_448_and_error_is_one_rounding():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((300, 512)).astype(np.float32)
    x[7] *= 1e-3
    x[8] *= 300.0
    codes, scale = f8.quantize_rows(x)
    assert codes.dtype == np.uint8 and scale.dtype == np.float32
    m, e = np.frexp(scale.astype(np.float64))
    assert np.all(m == 0.5)                                   # every scale a power of two
    top = np.max(np.abs(x.astype(np.float64)), axis=1) / scale
    assert np.all((top > 224) & (top <= 448))
    deq = f8.dequantize_rows(codes, scale)
    # one rounding to 3 mantissa bits: at most half a unit in the last place, i.e.
    # 2^-4 of the value in the normal range, 2^-10 * scale below it (the subnormal step)
    err = np.abs(deq - x.astype(np.float64))
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * scale[:, None].astype(np.float64))
    assert np.all(err <= bound)
    assert np.all(np.sign(deq) * np.sign(x) >= 0)
    # planted mistake: the old amax / 448 scale is not a power of two, and a scale one
    # binade too small saturates the row maximum
    assert not np.all(np.frexp(np.max(np.abs(x), axis=1) / 448.0)[0] == 0.5)
    assert np.any(top * 2 > 448)


def test_zero_row_tiny_and_huge_rows():
    codes, scale = f8.quantize_rows(np.zeros((2, 16), np.float32))
    assert np.all(codes == 0) and np.all(scale == 1.0)
    row = np.zeros((1, 16), np.float32)
    row[0, 3] = -2.0 ** -100                   # one nonzero element: -256 * 2^-108
    codes, scale = f8.quantize_rows(row)
    assert scale[0] == 2.0 ** -108 and codes[0, 3] == 0xF8
    assert f8.dequantize_rows(codes, scale)[0, 3] == -2.0 ** -100
    row[0, 3] = 2.0 ** -133                    # below the clamp: scale 2^-124, the smallest
    codes, scale = f8.quantize_rows(row)       # subnormal code 2^-9 (and bf16's smallest)
    assert scale[0] == 2.0 ** -124 and codes[0, 3] == 0x01 and codes[0, 2] == 0
    row[0, 3] = 3.0e38                         # past the upper clamp: saturates to 448
    codes, scale = f8.quantize_rows(row)
    assert scale[0] == 2.0 ** 117 and codes[0, 3] == 0x7E


def test_dequantized_cache_rows_keep_the_rope_part():
    rng = np.random.default_rng(2)
    rows = rng.standard_normal((70, 576)).astype(np.float32)
    out = f8.dequantized_cache_rows(rows, 512)
    assert np.array_equal(out[:, 512:], rows[:, 512:].astype(np.float64))
    codes, scale = f8.quantize_rows(rows[:, :512])
    assert np.array_equal(out[:, :512], f8.dequantize_rows(codes, scale))
