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


# ---------------------------------------------------- stochastic rounding --
# Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
# as 1, 2, 3", SC 2011): a counter-based generator, the published constants
# and round function.  Used for stochastic rounding of a 16-bit state (blog
# "The precision argument, derived": the recurrence copy kept in FP16 with
# stochastic rounding); the GPU path implements the same definition.
_PH_M0, _PH_M1 = np.uint64(0xD2E7470EE14C6C93), np.uint64(0xCA5A826395121157)
_PH_W0, _PH_W1 = np.uint64(0x9E3779B97F4A7C15), np.uint64(0xBB67AE8584CAA73B)
_M32 = np.uint64(0xFFFFFFFF)


def _mulhilo64(a, b):
    """Full 64 x 64 -> 128-bit product of uint64 arrays: (hi, lo)."""
    a = np.asarray(a, np.uint64)
    b = np.asarray(b, np.uint64)
    s32 = np.uint64(32)
    a_lo, a_hi = a & _M32, a >> s32
    b_lo, b_hi = b & _M32, b >> s32
    ll = a_lo * b_lo
    lh = a_lo * b_hi
    hl = a_hi * b_lo
    hh = a_hi * b_hi
    mid = (ll >> s32) + (lh & _M32) + (hl & _M32)
    lo = (ll & _M32) | ((mid & _M32) << s32)
    hi = hh + (lh >> s32) + (hl >> s32) + (mid >> s32)
    return hi, lo


def philox4x64(counter, key):
    """Philox4x64-10 of counters [..., 4] uint64 under keys [..., 2] uint64
    (broadcast); returns [..., 4] uint64."""
    c = np.array(np.broadcast_to(np.asarray(counter, np.uint64), np.broadcast_shapes(
        np.shape(counter), np.shape(key)[:-1] + (4,))), dtype=np.uint64)
    k = np.array(np.broadcast_to(np.asarray(key, np.uint64), c.shape[:-1] + (2,)), dtype=np.uint64)
    c0, c1, c2, c3 = (c[..., i].copy() for i in range(4))
    k0, k1 = k[..., 0].copy(), k[..., 1].copy()
    with np.errstate(over="ignore"):
        for rnd in range(10):
            if rnd:
                k0 = k0 + _PH_W0
                k1 = k1 + _PH_W1
            hi0, lo0 = _mulhilo64(_PH_M0, c0)
            hi1, lo1 = _mulhilo64(_PH_M1, c2)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return np.stack([c0, c1, c2, c3], axis=-1)


F16_MAX = 65504.0


SR_BITS = 16   # width of the random word one stochastic rounding consumes


def sr_f16(x, r) -> np.ndarray:
    """Stochastic rounding of real values x to fp16 with 16-bit random words r
    (same shape): |x| lies between two neighbouring fp16 values lo <= |x| < hi;
    the result is hi (with x's sign) when r < p 2^16, p = (|x| - lo) / (hi - lo),
    else lo, so it rounds up with probability ceil(p 2^16) / 2^16: exactly p
    when p is a multiple of 2^-16, as it is for every fp32 value from 2^-17
    up (at most 13 bits lie below the fp16 grid there), so E[result] = x for
    them.  Values that are fp16 already are unchanged; |x| >= 65504 and
    non-finite values round to nearest even (no stochastic choice at the top
    of the range)."""
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    a = np.abs(x)
    with np.errstate(over="ignore", invalid="ignore"):
        h = a.astype(np.float16)
    lo = h.astype(np.float64)
    hb = h.view(np.uint16)
    down = lo > a
    lo_b = np.where(down, hb - 1, hb).astype(np.uint16)
    lo = lo_b.view(np.float16).astype(np.float64)
    hi = (lo_b + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = (a - lo) / (hi - lo)
    up = r < np.ldexp(p, SR_BITS)
    mag = np.where(up, hi, lo)
    with np.errstate(over="ignore", invalid="ignore"):
        rne = x.astype(np.float16).astype(np.float64)
    out = np.where(np.isfinite(x) & (a < F16_MAX), np.copysign(mag, x), rne)
    return out


def sr_words(key, step, tile, n_elems):
    """The 16-bit random word for each of n_elems consecutive state elements
    (row-major d_v x d_k) of one tile at one step: element e uses word e % 16
    of Philox4x64-10 block (step, tile, e // 16, 0), whose four 64-bit outputs
    are split into 16-bit words least significant first (output 0 bits 0-15,
    16-31, 32-47, 48-63, then output 1, ...).  key: two uint64."""
    n_blk = (n_elems + 15) // 16
    ctr = np.zeros((n_blk, 4), np.uint64)
    ctr[:, 0] = np.uint64(step)
    ctr[:, 1] = np.uint64(tile)
    ctr[:, 2] = np.arange(n_blk, dtype=np.uint64)
    out = philox4x64(ctr, np.asarray(key, np.uint64))       # [n_blk, 4] uint64
    shifts = np.arange(4, dtype=np.uint64) * np.uint64(16)
    words = (out[..., None] >> shifts) & np.uint64(0xFFFF)  # [n_blk, 4 outputs, 4 half-words]
    return words.reshape(-1)[:n_elems]
