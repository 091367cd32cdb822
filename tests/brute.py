"""Pure-Python brute force and exact-arithmetic helpers for tiny inputs.

Independent of both the oracle and the HIP library: nothing here imports
either.  Used to pin the oracle (subset enumeration for masks, exact rational
means and roundings, integer dot products).
"""
from __future__ import annotations

import itertools
import math
import struct
from fractions import Fraction

import numpy as np


def f32(x) -> float:
    """Round a Python float to the nearest float32 (returns a Python float)."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def round_half_even(q: Fraction) -> int:
    fl = math.floor(q)
    rem = q - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def exact_to_float(q: Fraction, mant_bits: int = 24, emin: int = -126) -> float:
    """Round an exact rational to the nearest binary float with ``mant_bits``
    significand bits (ties to even), gradual underflow below 2**emin.
    mant_bits=24/emin=-126 is float32, 8/-126 is bfloat16.  No overflow
    handling (not needed here)."""
    if q == 0:
        return 0.0
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # fix e so that 2**e <= a < 2**(e+1)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - (mant_bits - 1))
    k = round_half_even(a / ulp)
    return sign * float(k * ulp)


def exact_to_f32(q: Fraction) -> float:
    return exact_to_float(q, 24, -126)


def exact_to_bf16(q: Fraction) -> float:
    return exact_to_float(q, 8, -126)


def beats(ak: float, k: int, aj: float, j: int) -> bool:
    """k beats j: larger magnitude, or equal magnitude and lower index."""
    return ak > aj or (ak == aj and k < j)


def brute_mask_group(vals, n: int):
    """Enumerate all n-subsets of a group; return the unique subset whose
    every kept element beats every dropped element."""
    m = len(vals)
    a = [abs(float(v)) for v in vals]
    found = []
    for S in itertools.combinations(range(m), n):
        rest = [j for j in range(m) if j not in S]
        if all(beats(a[i], i, a[j], j) for i in S for j in rest):
            found.append(set(S))
    assert len(found) == 1, (vals, found)
    return found[0]


def brute_mask(W: np.ndarray, n: int, m: int) -> np.ndarray:
    """Boolean [rows, cols] mask by subset enumeration."""
    rows, cols = W.shape
    out = np.zeros((rows, cols), dtype=bool)
    for r in range(rows):
        for g in range(cols // m):
            S = brute_mask_group(W[r, g * m:(g + 1) * m], n)
            for j in S:
                out[r, g * m + j] = True
    return out


def unpack_bits(mask_bits: np.ndarray, rows: int, cols: int) -> np.ndarray:
    bits = np.unpackbits(np.asarray(mask_bits, dtype=np.uint8), bitorder="little")
    return bits[: rows * cols].reshape(rows, cols).astype(bool)


def exact_mean_abs(row) -> Fraction:
    return sum((Fraction(abs(float(v))) for v in row), Fraction(0)) / len(row)


def brute_dot(a, b) -> int:
    return sum(int(x) * int(y) for x, y in zip(a, b))
