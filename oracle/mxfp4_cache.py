"""Plain CPU definitions of the MXFP4 latent cache -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import or run anything in ``oracle/``; the product never does, and this module
imports nothing from the product package.

Source: P3 = www.nxmr.cn/news/151634 (MLA operators).  Its introduction lists a
4-bit (NVFP4) quantized gather of the latent cache among the operators, and its §5
describes that gather's failure mode: 16-byte (uint4) vector loads of packed 4-bit values,
whose element offset halved (two values per byte) must be a whole number of 16-byte
units, from a 16-byte-aligned page-table base.  The page gives no layout.  NVFP4 is
NVIDIA's variant; the 4-bit float format gfx950 converts natively is the OCP
microscaling format MXFP4, and that is this library's reading:

* Elements are FP4 E2M1: 1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit.  The
  eight magnitudes are 0, 0.5 (the one subnormal), 1, 1.5, 2, 3, 4, 6.  There is no
  infinity and no NaN.  Code c has sign c >> 3 and magnitude code c & 7.
* Each block of 32 consecutive latent elements of a token shares one scale, an E8M0
  byte s meaning 2^(s - 127) (s = 255 would be NaN).  Element value = E2M1(code) * 2^(s - 127).
* Quantization of a block x (values exact in bf16), after the OCP MX rule:
  e = floor(log2(amax)) - 2, where amax = max |x_i| and 2 is the exponent of E2M1's
  largest value (6 = 1.5 * 2^2).  e is clamped to [-126, 127]; an all-zero block takes
  e = -126.  The clamp at -126 is this library's reading: the MX rule allows -127, but the
  decoding kernel builds the float32 scale 2^e from the byte, and that must be a normal
  number.  For bf16 inputs e never exceeds 125.  The scale byte is e + 127, in 1 .. 252.
* code_i is the E2M1 value nearest to x_i / 2^e, ties to the even code (mantissa bit clear).
  Magnitudes past 6 saturate to 6; the sign bit is x_i's, so a negative value that
  rounds to zero gives code 8 (-0).  x_i / 2^e is exact in float64, and the code is
  decided there.
* The latent row of a token is 16 blocks: d_c / 2 bytes of packed codes (byte j holds
  element 2j in its low nibble and element 2j + 1 in its high nibble) and d_c / 32 scale
  bytes.  k_R stays bf16, as in the FP8 cache (P3 §4: reduced RoPE precision is what
  breaks the absorbed scores).

The decode over an MXFP4 cache is then the plain non-absorbed decode
(``mla_oracle.mla_decode``) over the dequantized rows [E2M1(code) * 2^e | k_R].
"""
from __future__ import annotations

import numpy as np

BLOCK = 32                        # elements per shared scale
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_MAX = 6.0
E2M1_EMAX = 2                     # exponent of the largest magnitude: 6 = 1.5 * 2^2
SCALE_EXP_MIN, SCALE_EXP_MAX = -126, 127


def e2m1_value(codes) -> np.ndarray:
    """float64 value of each 4-bit E2M1 code (0 .. 15), from its sign, exponent and
    mantissa fields: exponent 0 is the subnormal m/2, otherwise (1 + m/2) * 2^(e - 1)."""
    c = np.asarray(codes).astype(np.int64)
    if np.any((c < 0) | (c > 15)):
        raise ValueError("E2M1 codes are 4-bit")
    sign = np.where(c >> 3, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + m * 0.5) * np.power(2.0, e - 1))
    return sign * mag


def e2m1_round(y) -> np.ndarray:
    """E2M1 code (uint8, 0 .. 15) nearest to each value of y, ties to the even code,
    magnitudes past 6 saturating to 6; the sign bit is y's.  A plain search over the
    eight magnitudes.  y must be finite."""
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        raise ValueError("E2M1 has no NaN or infinity: the values must be finite")
    a = np.minimum(np.abs(y), E2M1_MAX)
    d = np.abs(a[..., None] - E2M1_MAGNITUDES)          # distance to every magnitude
    best = d.min(axis=-1, keepdims=True)
    cand = d == best                                     # one or two nearest codes
    even = cand & ((np.arange(8) & 1) == 0)
    code = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1))
    return (code | np.where(np.signbit(y), 8, 0)).astype(np.uint8)


def e8m0_value(s) -> np.ndarray:
    """float64 value 2^(s - 127) of each E8M0 scale byte; 255 is NaN."""
    s = np.asarray(s).astype(np.int64)
    return np.where(s == 255, np.nan, np.power(2.0, s - 127))


def block_exponent(amax) -> np.ndarray:
    """The shared exponent e of blocks with largest magnitude amax (see the module
    docstring): floor(log2(amax)) - 2, clamped to [-126, 127]; -126 for amax = 0."""
    amax = np.asarray(amax, dtype=np.float64)
    with np.errstate(divide="ignore"):
        fl = np.floor(np.log2(np.where(amax > 0, amax, 1.0)))
    # log2 of a power of two is exact; guard the floor against a value just below it
    fl = np.where(np.power(2.0, fl + 1) <= amax, fl + 1, fl)
    fl = np.where(np.power(2.0, fl) > amax, fl - 1, fl)
    e = np.where(amax > 0, fl - E2M1_EMAX, SCALE_EXP_MIN)
    return np.clip(e, SCALE_EXP_MIN, SCALE_EXP_MAX).astype(np.int64)


def quantize_rows(latent) -> tuple[np.ndarray, np.ndarray]:
    """MXFP4 quantization of latent rows [n, d_c] (d_c a multiple of 32, values exact in
    bf16): (packed codes uint8 [n, d_c / 2], scale bytes uint8 [n, d_c / 32])."""
    x = np.asarray(latent)
    n, d_c = x.shape
    if d_c % BLOCK:
        raise ValueError("d_c must be a multiple of 32")
    packed = np.empty((n, d_c // 2), np.uint8)
    scales = np.empty((n, d_c // BLOCK), np.uint8)
    step = 2048  # rows at a time (the same arithmetic, in pieces that fit memory)
    for r in range(0, n, step):
        blocks = x[r:r + step].astype(np.float64).reshape(-1, d_c // BLOCK, BLOCK)
        e = block_exponent(np.max(np.abs(blocks), axis=-1))      # [rows, d_c / 32]
        codes = e2m1_round(blocks / np.power(2.0, e)[..., None]).reshape(-1, d_c)
        packed[r:r + step] = codes[:, 0::2] | (codes[:, 1::2] << 4)
        scales[r:r + step] = e + 127
    return packed, scales


def unpack_codes(packed) -> np.ndarray:
    """4-bit codes [n, 2 m] from packed bytes [n, m]: element 2j from the low nibble of
    byte j, element 2j + 1 from its high nibble."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def dequantize_rows(packed, scales) -> np.ndarray:
    """float64 latent rows [n, d_c]: E2M1(code) * 2^(s - 127), one s per 32 elements."""
    vals = e2m1_value(unpack_codes(packed))
    n, d_c = vals.shape
    sc = e8m0_value(scales)                                       # [n, d_c / 32]
    return (vals.reshape(n, d_c // BLOCK, BLOCK) * sc[..., None]).reshape(n, d_c)


def dequantized_cache_rows(rows, d_c: int) -> np.ndarray:
    """A sequence's cache rows [L, d_c + d_R] as an MXFP4 cache holds them: the latent part
    quantized and dequantized, the k_R part unchanged.  float64."""
    rows = np.asarray(rows)
    packed, scales = quantize_rows(rows[:, :d_c])
    out = np.empty(rows.shape, dtype=np.float64)
    out[:, :d_c] = dequantize_rows(packed, scales)
    out[:, d_c:] = rows[:, d_c:]
    return out
