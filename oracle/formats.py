"""Storage formats of a read copy, in exact (float64) arithmetic.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (see the package docstring).

A two-precision checkpoint (blog "ReplaySSM: an SSM decoder that writes its
state once every 16 tokens", section "The precision argument, derived")
keeps a read copy that is one rounding of the recurrence copy.  This module
defines that rounding for each read format, and the largest error it can
make (half a unit in the last place), which is what bounds a non-flush
step's output error.

  f16, bf16   IEEE binary16 / bfloat16, round to nearest even (the libraries'
              casts).
  e4m3        OCP 8-bit floating point, E4M3 (Open Compute Project, "OCP
              8-bit Floating Point Specification (OFP8)", rev. 1.0): sign,
              4 exponent bits with bias 7, 3 mantissa bits; no infinities;
              S.1111.111 is NaN, so the largest finite magnitude is
              1.75 * 2^8 = 448; subnormals are m/8 * 2^-6.  Each state row
              (the d_k entries of one output component) carries a power-of-two
              scale 2^e: the stored codes are E4M3(x * 2^-e), rounded to
              nearest even, and the row reads back as code * 2^e.  e is the
              smallest integer with max|x| * 2^-e <= 448, and at least -100
              (so an all-zero or vanishing row gets a normal fp32 scale).  With
              a power-of-two scale the scaling is exact, so the only rounding
              decision is the E4M3 one.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_EXP = -100   # lower clamp of a row's scale exponent


# ---------------------------------------------------------------- E4M3 --
def e4m3_encode(y) -> np.ndarray:
    """E4M3 codes (uint8) of real values, round to nearest even.  Magnitudes
    above 448 saturate to 448 (the scale rule never produces them)."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    code = np.zeros(y.shape, dtype=np.int64)
    # subnormal range |y| < 2^-6: multiples of 2^-9; m = 8 is the smallest
    # normal, whose code is also 8
    sub = a < 2.0**-6
    code[sub] = np.rint(a[sub] * 2.0**9).astype(np.int64)
    # normal range: 2^E <= |y| < 2^(E+1) holds 8 steps of 2^(E-3); m = 16
    # carries into the next binade, which (E + 7) * 8 + (m - 8) absorbs
    nor = ~sub
    if np.any(nor):
        fr, ex = np.frexp(a[nor])          # a = fr * 2^ex, fr in [0.5, 1)
        E = ex.astype(np.int64) - 1
        m = np.rint(np.ldexp(a[nor], -(E - 3).astype(np.int32))).astype(np.int64)  # 8..16
        code[nor] = (E + 7) * 8 + (m - 8)
    code = np.minimum(code, 0x7E)
    code |= np.where(np.signbit(y), 0x80, 0)
    return code.astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    """Real values of E4M3 codes (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.int64)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0**-9, np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32)))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


def e4m3_row_exponent(x) -> np.ndarray:
    """Per row (last axis): the smallest e with max|x| * 2^-e <= 448, at
    least E4M3_MIN_EXP."""
    amax = np.abs(np.asarray(x, dtype=np.float64)).max(axis=-1)
    fr, ex = np.frexp(amax)                # amax = fr * 2^ex, fr in [0.5, 1)
    # amax = f 2^E with f = 2 fr in [1, 2): e = E - 8 if f <= 1.75, else E - 7
    e = (ex.astype(np.int64) - 1) - 8 + (fr > 0.875)
    e = np.where(amax > 0, e, E4M3_MIN_EXP)
    return np.maximum(e, E4M3_MIN_EXP)


def e4m3_quantize_rows(x):
    """(codes uint8 [..., n], exponents int64 [...]) of rows x [..., n]."""
    x = np.asarray(x, dtype=np.float64)
    e = e4m3_row_exponent(x)
    return e4m3_encode(np.ldexp(x, -e[..., None].astype(np.int32))), e


def e4m3_dequantize_rows(codes, e) -> np.ndarray:
    return np.ldexp(e4m3_decode(codes), np.asarray(e)[..., None].astype(np.int32))


# --------------------------------------------------------------- all ----
def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """One rounding of x into a read-copy format, returned as float64: fp16,
    bf16 (round to nearest even, the libraries' casts), fp32, or E4M3 with
    a power-of-two scale per row (last axis)."""
    if dtype == "f16":
        return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)
    if dtype == "bf16":
        import torch
        return torch.from_numpy(np.ascontiguousarray(x, np.float64)).to(torch.bfloat16).double().numpy()
    if dtype == "f32":
        return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)
    if dtype == "e4m3":
        return e4m3_dequantize_rows(*e4m3_quantize_rows(x))
    raise ValueError(dtype)


def half_ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Half a unit in the last place of each value's representation in
    `dtype`: the most that round_to can move it (E4M3: at the row's scale)."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "e4m3":
        e = e4m3_row_exponent(x)[..., None]
        y = np.abs(np.ldexp(x, -e.astype(np.int32)))
        _, ex = np.frexp(np.maximum(y, 2.0**-6))
        return np.ldexp(np.ones_like(y), ((ex - 1) - 4 + e).astype(np.int32))
    mant, emin = {"f16": (10, -14), "bf16": (7, -126), "f32": (23, -126)}[dtype]
    _, ex = np.frexp(np.maximum(np.abs(x), 2.0**emin))
    return np.ldexp(np.ones_like(x), ((ex - 1) - mant - 1).astype(np.int32))
