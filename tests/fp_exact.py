"""Exact-arithmetic helpers for pinning the oracle (test code; independent of oracle/).

``rne_f32(q)`` rounds an exact rational to the nearest binary32 with ties to even, written
from the IEEE 754 definition (not through ``float(Fraction)``, which rounds to binary64 first
and can double-round).
"""
from fractions import Fraction
import math

import numpy as np


def rne_f32(q):
    """Nearest float32 (ties to even) to the rational q, as a numpy float32."""
    q = Fraction(q)
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    # e = floor(log2(a)), from the bit lengths, then corrected
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                      # below the normal range the quantum stays 2^-149
    quantum = Fraction(2) ** (e - 23)
    m = a / quantum
    n = math.floor(m)
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * quantum
    if val >= Fraction(2) ** 128:
        return np.float32(sign * np.inf)
    return np.float32(sign * float(val))   # val has <= 24 significant bits: exact in float


def frac_of_f32(f):
    return Fraction(float(np.float32(f)))


def e4m3_table_torch():
    """float32 values of all 256 E4M3 codes, decoded by torch's float8_e4m3fn dtype."""
    import torch
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).float().numpy()


def e8m0_table_torch():
    import torch
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e8m0fnu).float().numpy()


def brute_e4m3_encode(f, table=None):
    """Nearest finite E4M3 code to float f, ties to the even code, saturating at +-448;
    the sign of the code follows the sign of f (so -tiny -> 0x80).  Brute force over codes."""
    table = e4m3_table_torch() if table is None else table
    f = np.float32(f)
    if np.isnan(f):
        return None
    neg = bool(np.signbit(f))
    a = Fraction(float(abs(f)))
    best = None
    for c in range(0x00, 0x7F):           # all finite non-negative codes (0x7F is NaN)
        d = abs(Fraction(float(table[c])) - a)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1] | (0x80 if neg else 0)
