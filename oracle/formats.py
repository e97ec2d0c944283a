"""Number formats of an NVFP4 weight, written from their definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name the formats but print neither table nor rounding rule
(TensorFold issue #308, section "The checkpoint": each weight is a 4-bit e2m1
code, scaled by one e4m3 byte per 16 inputs and one fp32 weight_scale_2 per
tensor). Readings taken here:

* e2m1 is the OCP FP4 element: sign, 2 exponent bits (bias 1), 1 mantissa bit,
  no Inf or NaN; magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* e4m3 is OCP FP8 E4M3 "fn": bias 7, subnormals, no Inf, NaN at S.1111.111,
  largest finite 448 (the 6*448 of the per-tensor scale rests on it).
* Encoding rounds to nearest, ties to the even code (IEEE default).
* e4m3 encode saturates to 448; e2m1 encode clamps to 6.
* The sign of an e2m1 code is the sign bit of the value (so -0.0 -> 0x8).
"""
from __future__ import annotations

import numpy as np


# ------------------------------------------------------------------ bf16 (O1)
def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32. bf16 is the top half of binary32, so
    the widening is exact: the 16 bits move to the high half, the low half is 0."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even.

    Adding 0x7FFF plus the lowest kept bit to the 32-bit pattern and keeping the
    top 16 bits rounds the dropped half to nearest with ties going to an even
    kept pattern; a carry out of the mantissa correctly bumps the exponent (and
    overflows to Inf at the top). NaN inputs stay NaN (quiet bit forced)."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if np.any(nan):
        r = np.where(nan, ((u >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16), r)
    return r


# --------------------------------------------------------- generic minifloat
def minifloat_decode(code, ebits: int, mbits: int, bias: int, special: str = "none") -> np.ndarray:
    """Value of a sign/exponent/mantissa code, as float64 (exact for <= 16-bit formats).

    Exponent field e, mantissa field m:
      e == 0: (m / 2^mbits) * 2^(1 - bias)        (subnormal)
      e >  0: (1 + m / 2^mbits) * 2^(e - bias)    (normal)
    special: "none" (every code finite), "fn" (only all-ones e and m is NaN),
             "ieee" (all-ones e is Inf for m == 0, NaN otherwise)."""
    c = np.asarray(code, dtype=np.int64)
    s = (c >> (ebits + mbits)) & 1
    e = (c >> mbits) & ((1 << ebits) - 1)
    m = c & ((1 << mbits) - 1)
    frac = m.astype(np.float64) / float(1 << mbits)
    mag = np.where(e == 0, frac * 2.0 ** (1 - bias), (1.0 + frac) * np.exp2((e - bias).astype(np.float64)))
    emax = (1 << ebits) - 1
    mmax = (1 << mbits) - 1
    if special == "fn":
        mag = np.where((e == emax) & (m == mmax), np.nan, mag)
    elif special == "ieee":
        mag = np.where(e == emax, np.where(m == 0, np.inf, np.nan), mag)
    return np.where(s == 1, -mag, mag)


# -------------------------------------------------------------- e2m1 (O2, O5)
E2M1_MAX = 6.0


def e2m1_decode(code) -> np.ndarray:
    """4-bit e2m1 code (low nibble) -> float64 value."""
    return minifloat_decode(np.asarray(code, dtype=np.int64) & 0xF, 2, 1, 1, "none")


# Representable e2m1 magnitudes in code order and the midpoints between neighbours.
_E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
_E2M1_MIDS = (_E2M1_MAGS[:-1] + _E2M1_MAGS[1:]) / 2.0   # 0.25 .. 5.0


def e2m1_encode(q) -> np.ndarray:
    """float32 q -> 4-bit e2m1 code (uint8), round to nearest, ties to even, clamp at 6.

    The magnitude index counts the midpoints that |q| passes: it moves past
    midpoint i (between index i and i+1) when |q| is above it, or exactly on it
    and index i+1 is even (mantissa bit 0). |q| >= 6 lands on index 7 (6.0)
    because every midpoint is passed. The sign bit is the sign bit of q."""
    q = np.asarray(q, dtype=np.float32)
    a = np.abs(q)                       # the midpoints are exact in float32
    idx = np.zeros(q.shape, dtype=np.uint8)
    for i, mid in enumerate(_E2M1_MIDS.astype(np.float32)):
        up_even = ((i + 1) % 2) == 0
        passed = (a > mid) | ((a == mid) & up_even)
        idx = idx + passed.astype(np.uint8)
    sign = np.signbit(q).astype(np.uint8)
    return (idx | (sign << 3)).astype(np.uint8)


# -------------------------------------------------------------- e4m3 (O3, O4)
E4M3_MAX = 448.0
E4M3_MAX_BYTE = 0x7E


def e4m3_decode(byte) -> np.ndarray:
    """e4m3fn byte -> float64 value (0x7F and 0xFF are NaN)."""
    return minifloat_decode(np.asarray(byte, dtype=np.int64) & 0xFF, 4, 3, 7, "fn")


def e4m3_encode(v) -> np.ndarray:
    """Non-negative finite float32 v -> e4m3fn byte, round to nearest even, saturating at 448.

    Below 2^-6 the grid is the subnormal one, multiples of 2^-9; at and above it,
    v = 2^e * (1 + f) and f is rounded to eighths, a rounding up to 8/8 carrying
    into the exponent. The subnormal grid rounding up to 8 * 2^-9 gives byte 0x08,
    which is exactly the smallest normal."""
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    if np.any(v < 0) or not np.all(np.isfinite(v)):
        raise ValueError("e4m3_encode expects finite non-negative values")
    out = np.empty(v.shape, dtype=np.int64)
    sub = v < 2.0 ** -6
    out[sub] = np.rint(v[sub] * 2.0 ** 9).astype(np.int64)          # rint: ties to even
    nv = v[~sub]
    mant, ex = np.frexp(nv)                 # nv = mant * 2^ex, mant in [0.5, 1)
    e = ex - 1                              # nv = (2*mant) * 2^e, 2*mant in [1, 2)
    m = np.rint((2.0 * mant - 1.0) * 8.0).astype(np.int64)
    carry = m == 8
    e = e + carry
    m = np.where(carry, 0, m)
    out[~sub] = ((e + 7) << 3) | m
    out = np.where(v >= E4M3_MAX, E4M3_MAX_BYTE, out)
    out = np.minimum(out, E4M3_MAX_BYTE)
    return out.astype(np.uint8)
