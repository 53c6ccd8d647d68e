"""Pins of the MXFP4 cache oracle (oracle/mxfp4_cache.py), CPU only.

The element format is pinned against the E2M1 value table of the OCP microscaling
specification (written out by hand here) and by brute force over the 16 codes; the
scale byte against torch's own float8_e8m0fnu type (an independent implementation of
E8M0); the quantizer against its defining properties (the block maximum lands in
[4, 8) before saturation, one rounding per element, zero and tiny blocks, the packing
order)."""
import numpy as np
import pytest
import torch

import oracle.mxfp4_cache as f4

CODES = np.arange(16, dtype=np.uint8)
# OCP MX E2M1 table: codes 0..7 are +0, 0.5, 1, 1.5, 2, 3, 4, 6; codes 8..15 the negatives
TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_values_match_the_table():
    v = f4.e2m1_value(CODES)
    assert list(v[:8]) == TABLE
    assert list(v[8:]) == [-t for t in TABLE]
    assert np.signbit(v[8]) and v[8] == 0.0                    # code 8 is -0


def test_e2m1_round_trip_of_every_code():
    got = f4.e2m1_round(f4.e2m1_value(CODES))
    assert np.array_equal(got, CODES)


def test_e2m1_round_is_the_nearest_value_by_brute_force():
    rng = np.random.default_rng(1)
    y = np.concatenate([rng.uniform(-7, 7, 20000), rng.standard_normal(5000) * 0.3])
    got = f4.e2m1_value(f4.e2m1_round(y))
    table = np.array(TABLE + [-t for t in TABLE])
    clipped = np.clip(y, -6, 6)
    best = np.min(np.abs(clipped[:, None] - table[None, :]), axis=1)
    assert np.allclose(np.abs(got - clipped), best, rtol=0, atol=0)


def test_e2m1_ties_go_to_the_even_code_and_saturate():
    # midpoints: 0.25 -> 0 (code 0), 0.75 -> 1.0 (code 2), 1.25 -> 1.0, 1.75 -> 2.0,
    # 2.5 -> 2.0, 3.5 -> 4.0, 5.0 -> 4.0 (code 6); past 6 -> 6
    y = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 1e30, -0.25, -5.0, -7.0]
    assert list(f4.e2m1_round(y)) == [0, 2, 2, 4, 4, 6, 6, 7, 7, 8, 14, 15]
    # just off the midpoints
    assert list(f4.e2m1_round([0.2500001, 0.7499999, 4.9999999, 5.0000001])) == [1, 1, 6, 7]
    with pytest.raises(ValueError):
        f4.e2m1_round([np.nan])


def test_e8m0_matches_torch_float8_e8m0fnu():
    s = np.arange(255, dtype=np.uint8)
    ref = torch.from_numpy(s.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(f4.e8m0_value(s), ref)
    assert np.isnan(f4.e8m0_value(255))


def test_block_exponent_by_hand():
    amax = np.array([1.0, 1.5, 2.0, 5.99, 6.0, 7.9, 8.0, 0.0, 2.0 ** -130, 3.0 * 2.0 ** 100])
    assert list(f4.block_exponent(amax)) == [-2, -2, -1, 0, 0, 0, 1, -126, -126, 99]


@pytest.mark.parametrize("seed", [0, 1])
def test_block_maximum_lands_in_4_to_8_and_error_is_one_rounding(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((64, 512)) * rng.uniform(0.01, 100, (64, 1))).astype(np.float32)
    packed, scales = f4.quantize_rows(x)
    e = scales.astype(np.int64) - 127
    blocks = x.astype(np.float64).reshape(64, 16, 32)
    q = blocks / np.power(2.0, e)[..., None]
    amax_q = np.max(np.abs(q), axis=-1)
    assert np.all((amax_q >= 4) & (amax_q < 8))
    deq = f4.dequantize_rows(packed, scales).reshape(64, 16, 32)
    err = np.abs(deq - blocks) / np.power(2.0, e)[..., None]
    # one E2M1 rounding: at most half a step (0.25 below 2, 0.5 in [2, 4], 1 in [4, 6]),
    # or the saturation from (6, 8) to 6
    step = np.where(np.abs(q) < 2, 0.5, np.where(np.abs(q) < 4, 1.0, 2.0))
    assert np.all((err <= step / 2) | (np.abs(q) > 6))
    assert np.all(np.abs(deq) <= 6 * np.power(2.0, e)[..., None])


def test_zero_tiny_and_negative_blocks():
    x = np.zeros((2, 64), np.float32)
    x[1, :32] = 2.0 ** -140                       # a block far below the smallest scale
    x[1, 32:] = -np.linspace(0, 3, 32)
    packed, scales = f4.quantize_rows(x)
    assert list(scales[0]) == [1, 1] and np.all(packed[0] == 0)
    assert scales[1, 0] == 1                      # clamped to 2^-126
    assert np.all(f4.dequantize_rows(packed, scales)[1, :32] == 0)
    deq = f4.dequantize_rows(packed, scales)[1, 32:]
    assert np.all(deq <= 0) and deq[-1] == -3.0   # amax 3 -> e = -1, 3 / 0.5 = 6 exactly


def test_packing_order():
    x = np.zeros((1, 32), np.float32)
    x[0, 0], x[0, 1], x[0, 2] = 6.0, -1.0, 0.5   # amax 6 -> e = 0
    packed, scales = f4.quantize_rows(x)
    assert scales[0, 0] == 127
    assert packed[0, 0] == 0x7 | (0x8 | 0x2) << 4   # element 0 low nibble, element 1 high
    assert packed[0, 1] == 0x1
    assert np.array_equal(f4.unpack_codes(packed)[0, :3], [7, 10, 1])


def test_dequantized_cache_rows_keep_the_rope_part():
    rng = np.random.default_rng(3)
    rows = rng.standard_normal((10, 576)).astype(np.float32)
    out = f4.dequantized_cache_rows(rows, 512)
    assert np.array_equal(out[:, 512:], rows[:, 512:].astype(np.float64))
    p, s = f4.quantize_rows(rows[:, :512])
    assert np.array_equal(out[:, :512], f4.dequantize_rows(p, s))


def test_planted_mistakes_fail_the_pins():
    """Each plausible slip in the quantizer fails one of the checks above: a block
    exponent off by one (the maximum leaves [4, 8)), ties to the odd code, or swapped
    nibbles."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((8, 64)).astype(np.float32)
    packed, scales = f4.quantize_rows(x)
    e = scales.astype(np.int64) - 127
    amax = np.max(np.abs(x.astype(np.float64).reshape(8, 2, 32)), axis=-1)
    assert np.all((amax / 2.0 ** (e + 1) < 4)) and np.all(amax / 2.0 ** (e - 1) >= 8)
    half_odd = [1, 3, 5, 5, 7]   # ties of 0.25, 1.25, 2.5, 3.5, 5 rounded to the odd code
    assert not np.array_equal(half_odd, f4.e2m1_round([0.25, 1.25, 2.5, 3.5, 5.0]))
    swapped = (packed >> 4) | ((packed & 0xF) << 4)
    assert not np.array_equal(f4.dequantize_rows(swapped, scales), f4.dequantize_rows(packed, scales))
