"""Plain CPU definitions of the FP8 (E4M3) latent cache -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import or run anything in ``oracle/``; the product never does, and this module
imports nothing from the product package.

Source: P3 = www.nxmr.cn/news/151634 (MLA operators).  Its introduction lists a
quantized (NVFP4) gather of the latent cache among the operators, and its §5 names the
gather's failure mode: the 16-byte vectorized loads need a 16-byte-aligned page-table
base and element offsets that are whole 16-byte units.  The page gives no format beyond
that, so the format here is this library's reading, on the 8-bit float format gfx950
converts natively:

* Each token's 512-d latent c_KV is stored as 8-bit E4M3 codes with one power-of-two
  scale per token, kept in a float32 slot: value = decode(code) * scale.  The 64-d RoPE key
  k_R stays bf16: it carries position, and P3 §4 warns that reduced precision in the RoPE
  part is what breaks the absorbed scores.
* E4M3 ("fn" variant, as in the OCP 8-bit float specification): 1 sign bit, 4 exponent
  bits with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals m/8 * 2^-6;
  no infinities; 0x7F and 0xFF are NaN; the largest finite value is 448.
* Quantization of a row x (its values exact in bf16): amax = max |x_i|; scale = 2^e with
  e the smallest integer such that amax <= 448 * 2^e, clamped to [-124, 117] (e = 0 for
  an all-zero row); code_i = the E4M3 value nearest to x_i / scale (an exact quotient),
  ties to the even code, magnitudes past 448 saturating to 448.  The scale is a power of
  two so that every decode(code) * scale is exact in bf16: the decoding kernel converts
  code and scale in one exact step.  E4M3's relative precision is the same in every
  binade, so a power-of-two scale costs at most one binade at the low end of the range;
  the row maximum lands in (224, 448].  The clamps keep 448 * scale below bf16's largest
  value and every subnormal E4M3 value times the scale on bf16's subnormal grid.

The decode over an FP8 cache is then the plain non-absorbed decode
(``mla_oracle.mla_decode``) over the dequantized rows [decode(code) * scale | k_R].
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN = 0x7F


def e4m3_value(codes) -> np.ndarray:
    """float64 value of each E4M3 code (uint8), from its sign, exponent and mantissa."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.power(2.0, e - 7))
    out = sign * mag
    return np.where((e == 15) & (m == 7), np.nan, out)


# The non-negative finite codes 0x00 .. 0x7E in increasing order of value.
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALUES = e4m3_value(_POS_CODES)


def e4m3_round(x) -> np.ndarray:
    """E4M3 code (uint8) nearest to each value of x, ties to the even code (mantissa
    bit 0 clear), magnitudes past 448 saturating to 448, NaN to 0x7F; the sign bit is
    x's (so -0.0 and negative values that round to zero give 0x80).  A plain search over
    the table of representable values."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 0, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((_POS_CODES[hi] & 1) == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    code = np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(E4M3_NAN), code).astype(np.uint8)


SCALE_EXP_MIN, SCALE_EXP_MAX = -124, 117


def scale_exponent(amax) -> np.ndarray:
    """The smallest integer e with amax <= 448 * 2^e, clamped to [-124, 117]; 0 where amax
    is 0.  amax is float64 here, so the comparisons are exact."""
    amax = np.asarray(amax, dtype=np.float64)
    pos = amax > 0
    with np.errstate(divide="ignore"):
        e = np.ceil(np.log2(np.where(pos, amax, E4M3_MAX) / E4M3_MAX))
    # settle the rounding of log2 with exact comparisons against 448 * 2^e
    e = np.where(E4M3_MAX * np.power(2.0, e) < amax, e + 1, e)
    e = np.where(E4M3_MAX * np.power(2.0, e - 1) >= amax, e - 1, e)
    e = np.clip(e, SCALE_EXP_MIN, SCALE_EXP_MAX)
    return np.where(pos, e, 0).astype(np.int64)


def quantize_rows(latent) -> tuple[np.ndarray, np.ndarray]:
    """Per-token E4M3 quantization of latent rows [n, d_c] (values exact in bf16):
    (codes uint8 [n, d_c], scales float32 [n], each a power of two) as defined in the
    module docstring."""
    x = np.asarray(latent, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1).astype(np.float64)
    e = scale_exponent(amax)
    scale = np.power(2.0, e).astype(np.float32)
    codes = np.empty(x.shape, np.uint8)
    step = 4096  # rows at a time (the same arithmetic, in cache-sized pieces)
    for r in range(0, x.shape[0], step):
        q = x[r:r + step].astype(np.float64) / np.power(2.0, e[r:r + step])[:, None]
        codes[r:r + step] = e4m3_round(q)
    return codes, scale


def dequantize_rows(codes, scales) -> np.ndarray:
    """float64 latent rows [n, d_c]: decode(code) * scale."""
    return e4m3_value(codes) * np.asarray(scales, dtype=np.float64)[..., None]


def dequantized_cache_rows(rows, d_c: int) -> np.ndarray:
    """A sequence's cache rows [L, d_c + d_R] as an FP8 cache holds them: the latent part
    quantized and dequantized, the k_R part unchanged.  float64."""
    rows = np.asarray(rows)
    codes, scales = quantize_rows(rows[:, :d_c])
    out = np.empty(rows.shape, dtype=np.float64)
    out[:, :d_c] = dequantize_rows(codes, scales)
    out[:, d_c:] = rows[:, d_c:]
    return out
