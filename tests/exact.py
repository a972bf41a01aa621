"""Exact-arithmetic helpers for the tests (independent of the oracle and of
the GPU library): rational rounding to binary float formats and format
decoding from the golden tables."""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_e2m1_table() -> list[float]:
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                c, v = line.split()
                vals[int(c)] = float(v)
    return [vals[c] for c in range(16)]


def round_fraction(s: Fraction, sig_bits: int, min_exp: int = -126) -> Fraction:
    """Nearest value (ties to even) of the exact rational ``s`` in a binary
    format with ``sig_bits`` significant bits and smallest normal exponent
    ``min_exp`` (subnormals kept, no overflow handling)."""
    if s == 0:
        return Fraction(0)
    a = abs(s)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e, min_exp) - (sig_bits - 1)
    r = round(a / Fraction(2) ** q)  # Fraction rounding is half-to-even
    v = Fraction(r) * Fraction(2) ** q
    return v if s > 0 else -v


def fp32_of(s: Fraction) -> np.float32:
    return np.float32(float(round_fraction(s, 24)))


def bf16_bits_of(s: Fraction) -> int:
    v = np.float32(float(round_fraction(s, 8)))
    return int(np.array([v], np.float32).view(np.uint32)[0] >> 16)


def bf16_to_f64(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(a) -> np.ndarray:
    """Vectorised RNE of doubles to bf16 through exact Fractions (slow; small
    arrays only)."""
    a = np.asarray(a, np.float64)
    return np.array([bf16_bits_of(Fraction(float(v))) for v in a.ravel()],
                    np.uint16).reshape(a.shape)


def mxfp4_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[rows][cols/2] code bytes + [rows][cols/32] scale bytes -> [rows][cols]
    float64, decoding codes through the golden E2M1 table and scales as
    2^(b-127) (byte 255 -> NaN). Column 2j sits in the low nibble of byte j."""
    table = np.array(load_e2m1_table())
    lo = codes & 0x0F
    hi = codes >> 4
    vals = np.empty((codes.shape[0], codes.shape[1] * 2))
    vals[:, 0::2] = table[lo]
    vals[:, 1::2] = table[hi]
    sc = np.where(scales == 255, np.nan, np.ldexp(1.0, scales.astype(np.int64) - 127))
    return vals * np.repeat(sc, 32, axis=1)
