"""Output encodings of compressed entries, written from their definitions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

* bfloat16: 1 sign, 8 exponent (bias 127), 7 stored mantissa bits;
  round to nearest, ties to even.
* FP8 E4M3 in the OCP 8-bit floating point format ("E4M3FN"): 1 sign,
  4 exponent bits (bias 7), 3 mantissa bits; no infinities; the single NaN
  pattern per sign is S.1111.111, so the largest finite value is
  1.75 * 2^8 = 448; exponent field 0 holds subnormals m * 2^-9.
  Encoding rounds to nearest, ties to even, and saturates to +-448.
* Per-entry scale (the fp8 KV storage that "混合压缩注意力双方案解析" names in
  its section on mixed-precision storage; the scale rule itself is this
  library's reading): s_i = max_ch |x[i, ch]| / 448, or 1 for an all-zero row;
  the stored code is encode(x[i, ch] / s_i).
"""

from __future__ import annotations

import numpy as np

FP8_E4M3_MAX = 448.0


def _round_to_step(x: np.ndarray, mant_bits: int, min_exp: int) -> np.ndarray:
    """Round float64 x to `mant_bits` stored mantissa bits, RNE.

    The spacing of representable values around |x| is 2^(e - mant_bits) where
    e = floor(log2 |x|), but never finer than 2^(min_exp - mant_bits)
    (subnormal range).  Division by a power of two is exact in float64, and
    np.rint rounds halfway cases to even.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    with np.errstate(divide="ignore"):
        _, E = np.frexp(ax)              # ax = f * 2^E, 0.5 <= f < 1  ->  e = E - 1
    e = np.maximum(E - 1, min_exp)
    step = np.ldexp(1.0, e - mant_bits)
    return np.sign(x) * np.rint(ax / step) * step


def round_bf16(x) -> np.ndarray:
    """Nearest bfloat16 value (ties to even), returned as float64.

    Range handling: finite inputs only (the compressor's outputs are convex
    combinations of finite inputs); the minimum normal exponent is -126.
    """
    return _round_to_step(x, mant_bits=7, min_exp=-126)


def fp8_e4m3_decode(codes) -> np.ndarray:
    """Value of each OCP E4M3FN code (uint8) as float64; NaN codes give NaN."""
    codes = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(codes & 0x80, -1.0, 1.0)
    ef = (codes >> 3) & 0xF
    mf = codes & 0x7
    normal = np.ldexp(1.0 + mf / 8.0, ef - 7)
    sub = np.ldexp(mf.astype(np.float64), -9)
    val = np.where(ef == 0, sub, normal)
    val = np.where((ef == 15) & (mf == 7), np.nan, val)
    return sign * val


def fp8_e4m3_encode(x) -> np.ndarray:
    """OCP E4M3FN code (uint8) of float64 x: saturate to +-448, RNE.

    The rounded magnitude q is a multiple of 2^(e-3) (e >= -6) and at most
    448, so it maps back to fields exactly: subnormal codes hold q / 2^-9,
    normal codes hold exponent e + 7 and mantissa (q / 2^e - 1) * 8.
    A NaN input is rejected; the compressor never produces one.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.isnan(x)):
        raise ValueError("NaN has no saturating E4M3 encoding here")
    xc = np.clip(x, -FP8_E4M3_MAX, FP8_E4M3_MAX)
    q = np.abs(_round_to_step(xc, mant_bits=3, min_exp=-6))
    q = np.minimum(q, FP8_E4M3_MAX)                 # rounding near 448 stays <= 448
    with np.errstate(divide="ignore"):
        _, E = np.frexp(q)
    e = E - 1
    is_sub = q < 2.0 ** -6
    sub_code = np.rint(q / 2.0 ** -9).astype(np.int64)
    e_safe = np.where(is_sub, 0, e)
    mant = np.rint((np.ldexp(q, -e_safe) - 1.0) * 8.0).astype(np.int64)
    norm_code = ((e_safe + 7) << 3) | mant
    code = np.where(is_sub, sub_code, norm_code)
    code = np.where(np.signbit(xc), code | 0x80, code)    # -0 keeps its sign bit
    return code.astype(np.uint8)


def fp8_entry_quantize(X):
    """Per-entry scaled E4M3 encoding of entries X (E x c), float64.

    Returns (codes uint8 (E x c), scales float64 (E,)) with
    s_i = max_ch |X_i| / 448 (1 if the row is all zero) and
    codes = encode(X_i / s_i).  Decoding is decode(code) * s_i.
    """
    X = np.asarray(X, dtype=np.float64)
    amax = np.abs(X).max(axis=1) if X.shape[1] else np.zeros(X.shape[0])
    scales = np.where(amax > 0, amax / FP8_E4M3_MAX, 1.0)
    return fp8_e4m3_encode(X / scales[:, None]), scales
