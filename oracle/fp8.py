"""FP8 (E4M3) weight quantisation, as the oracle reads it (NumPy).

TEST INFRASTRUCTURE ONLY, like the rest of this package.

The codemajin.net explainer's step timings (§5.2) are measured at FP8
precision, and a news page puts the quantised model in 18 GB; neither gives
the format. The reading taken here:

  * element format: OCP 8-bit floating point E4M3 ("e4m3fn"): 1 sign bit,
    4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
    subnormals m * 2^-9; the largest finite value is 448 (field 15, mantissa
    6); 0x7f / 0xff are NaN and never produced; no infinities;
  * rounding: to nearest, ties to even mantissa;
  * scaling: one power of two per weight row (output channel), 2^e with the
    smallest integer e such that max_k |W[n][k]| <= 448 * 2^e (e = 0 for an
    all-zero row), so W[n][k] * 2^-e is exact and never exceeds 448;
  * dequantised weight: decode(code) * 2^e, exact in float64 (and in bf16).

Parity status: pinned by the decode table's closed form, torch's own
float8_e4m3fn conversion, the round trip of every finite code, the
ties-to-even cases and the half-ulp error bound (tests/test_oracle_pins.py).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code (uint8) as float64: (-1)^s * 2^(E-7) * (1 + m/8)
    for exponent field E >= 1, (-1)^s * m * 2^-9 for E = 0."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    E = (c >> 3) & 15
    m = c & 7
    normal = np.ldexp(1.0 + m / 8.0, (E - 7).astype(np.int64))
    sub = m * 2.0 ** -9
    v = s * np.where(E > 0, normal, sub)
    if np.any((c & 0x7F) == 0x7F):
        raise ValueError("NaN code")
    return v


def e4m3_encode(v) -> np.ndarray:
    """E4M3 code of each value (|v| <= 448, finite), rounded to nearest with
    ties to even. Below 2^-6 the step is 2^-9 (subnormals); in [2^E, 2^(E+1))
    it is 2^(E-3). The sign bit follows the value's sign (also for zero)."""
    v = np.asarray(v, np.float64)
    if np.any(~np.isfinite(v)) or np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("value outside the E4M3 range")
    sign = np.signbit(v).astype(np.int64)
    a = np.abs(v)
    code = np.zeros(a.shape, np.int64)
    sub = a < 2.0 ** -6
    # subnormal range: multiples of 2^-9; a result of 8 is the smallest normal
    # (field 1, mantissa 0), whose code is also 8
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)
    nz = ~sub
    _, x = np.frexp(a[nz])  # a = f * 2^x, f in [0.5, 1): floor(log2 a) = x - 1
    E = x - 1
    q = np.rint(np.ldexp(a[nz], 3 - E)).astype(np.int64)  # in [8, 16]
    carry = q == 16
    E = np.where(carry, E + 1, E)
    q = np.where(carry, 8, q)
    code[nz] = ((E + 7) << 3) | (q - 8)
    return ((sign << 7) | code).astype(np.uint8)


def row_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2^e (0 where amax == 0)."""
    amax = np.asarray(amax, np.float64)
    f, x = np.frexp(amax)  # amax = f * 2^x, f in [0.5, 1); 448 = 0.875 * 2^9
    e = np.where(f <= 0.875, x - 9, x - 8)
    return np.where(amax == 0, 0, e).astype(np.int64)


def quantize_rows(W) -> tuple:
    """codes uint8 [N][K] and row exponents int [N] of a weight matrix W [N][K]."""
    W = np.asarray(W, np.float64)
    e = row_exponent(np.abs(W).max(axis=1))
    codes = e4m3_encode(np.ldexp(W, -e[:, None]))
    return codes, e


def dequantize_rows(codes, e) -> np.ndarray:
    """float64 weights decode(codes) * 2^e, row by row."""
    return np.ldexp(e4m3_decode(codes), np.asarray(e, np.int64)[:, None])


def dequantize_bank(W) -> np.ndarray:
    """Quantise then dequantise a weight bank [..., N, K] row by row: the
    weights an FP8 expert actually multiplies with."""
    W = np.asarray(W, np.float64)
    flat = W.reshape(-1, W.shape[-1])
    codes, e = quantize_rows(flat)
    return dequantize_rows(codes, e).reshape(W.shape)
