"""Pins of the oracle's linear output modes (CPU): O14a (bf16 encoding of a real number) and
O14 (a linear of the head's own layers: fp32, bf16, or bf16 of a residual plus the sum),
from "dsv41 Zig: the TFE draft head (TF_DS_DRAFTER=eagle), off by default", commit notes on
the own GEMV.

 * O14a against torch's float32 -> bfloat16 conversion (a library routine) on float32
   values of every class, and against closed forms: ties to even, a single rounding from
   the double (which a float32 detour would break), subnormals and the overflow threshold;
 * O14 mode 0 against O5 bit for bit; modes 1 and 2 against exact rational arithmetic
   (Python fractions) with round-half-even written here, on small inputs of each format;
 * a planted mistake: rounding the sum to bf16 before the residual add (two roundings)
   must give a different answer on a constructed case.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth


def torch_bf16(f32):
    t = torch.from_numpy(np.asarray(f32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_encode_matches_torch_on_floats():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32)
    # halfway and near-halfway patterns, subnormals, values at the overflow edge
    low = np.array([0x8000, 0x7fff, 0x8001, 0x18000, 0x0, 0xffff], np.uint32)
    hi = rng.integers(0, 2**16, 500).astype(np.uint32) << 16
    bits = np.concatenate([bits, (hi[:, None] | low[None, :]).ravel(),
                           np.array([0x7f7f8000, 0x7f7f7fff, 0x7f7fffff, 0x00008000,
                                     0x00018000, 0x80008000, 0x7f800000, 0xff800000],
                                    np.uint32)])
    f = bits.view(np.float32)
    f = f[~np.isnan(f)]
    want = torch_bf16(f)
    got = np.array([oracle.bf16_encode(float(v)) for v in f], np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(f.view(np.uint32)[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


@pytest.mark.parametrize("d,bits", [
    (1.0, 0x3f80),
    (1 + 2**-8, 0x3f80),                  # halfway: to the even neighbour 1.0
    (1 + 3 * 2**-8, 0x3f82),              # halfway: to the even neighbour 1 + 2^-6
    (1 + 2**-8 + 2**-40, 0x3f81),         # above halfway in the double (a float would lose it)
    (-(1 + 2**-8 + 2**-40), 0xbf81),
    (2.0**-133, 0x0001),                  # the least subnormal
    (2.0**-134, 0x0000),                  # halfway to zero: even
    (1.5 * 2.0**-134, 0x0001),
    ((2 - 2**-7) * 2.0**127, 0x7f7f),     # the largest finite
    ((2 - 2**-8) * 2.0**127, 0x7f80),     # halfway above it: to even, which is infinity
    (-0.0, 0x8000),
    (float("nan"), 0x7fc0),
])
def test_bf16_encode_closed_forms(d, bits):
    assert oracle.bf16_encode(d) == bits


def _bf16_frac(b):
    return Fraction(float(np.uint32(int(b) << 16).view(np.float32)))


def _rne_bf16_exact(v):
    """Round a rational to bf16 bits, ties to even (written from the format's definition)."""
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e - 7, -133)
    n = a / Fraction(2) ** q
    fl = n.numerator // n.denominator
    rem = n - fl
    r = fl + (1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2) else 0)
    val = r * Fraction(2) ** q
    if val >= Fraction(2) ** 128:
        return sign | 0x7f80
    f = np.float32(float(val))
    return sign | int(f.view(np.uint32) >> 16)


def _exact_dot_rows(fmt, w, scale, x):
    N, K = w.shape
    R = x.shape[0]
    xv = [[_bf16_frac(x[r, k]) for k in range(K)] for r in range(R)]
    out = np.empty((R, N), dtype=object)
    for n in range(N):
        wv = [Fraction(oracle.e4m3_value(w[n, k])) if fmt != oracle.FMT_BF16 else
              _bf16_frac(w[n, k]) for k in range(K)]
        if fmt == oracle.FMT_FP8_ROW:
            wv = [v * Fraction(float(scale[n])) for v in wv]
        elif fmt == oracle.FMT_FP8_BLOCK32:
            wv = [v * Fraction(oracle.e8m0_value(scale[n // 32, k // 32])) for k, v in
                  enumerate(wv)]
        for r in range(R):
            out[r, n] = sum(a * b for a, b in zip(xv[r], wv))
    return out


@pytest.mark.parametrize("fmt", [oracle.FMT_BF16, oracle.FMT_FP8_BLOCK32, oracle.FMT_FP8_ROW])
def test_linear_modes_exact_on_small_inputs(fmt):
    N, K, R = 40, 64, 3
    w = synth.random_head(N, K, seed=11 + fmt, std=0.05)
    x = synth.random_acts(R, K, seed=12 + fmt)
    scale = None
    if fmt == oracle.FMT_FP8_BLOCK32:
        w, scale = oracle.quant_block32(w)
    elif fmt == oracle.FMT_FP8_ROW:
        w, scale = oracle.quant_row(w)
    res = synth.random_acts(R, N, seed=13 + fmt)
    exact = _exact_dot_rows(fmt, w, scale, x)
    f32 = oracle.linear(fmt, w, scale, x, oracle.MODE_F32)
    assert np.array_equal(f32.view(np.uint32), oracle.gemv(fmt, w, scale, x).view(np.uint32))
    b16 = oracle.linear(fmt, w, scale, x, oracle.MODE_BF16)
    add = oracle.linear(fmt, w, scale, x, oracle.MODE_ADD_BF16, res)
    for r in range(R):
        for n in range(N):
            assert b16[r, n] == _rne_bf16_exact(exact[r, n]), (r, n)
            assert add[r, n] == _rne_bf16_exact(_bf16_frac(res[r, n]) + exact[r, n]), (r, n)


def test_control_two_roundings_fail():
    """residual 1.0 plus a sum of 2^-8 + 2^-30: one rounding gives 1 + 2^-7, rounding the sum
    to bf16 first (2^-8) and then the add (a tie, to even) gives 1.0."""
    K = 32
    x = np.zeros((1, K), np.uint16)
    x[0, 0] = np.float32(2.0**-8).view(np.uint32) >> 16
    x[0, 1] = np.float32(2.0**-30).view(np.uint32) >> 16
    w = np.zeros((1, K), np.uint16)
    w[0, :2] = np.float32(1.0).view(np.uint32) >> 16
    res = np.array([[np.float32(1.0).view(np.uint32) >> 16]], np.uint16)
    good = oracle.linear(oracle.FMT_BF16, w, None, x, oracle.MODE_ADD_BF16, res)
    assert good[0, 0] == 0x3f81
    s = oracle.linear(oracle.FMT_BF16, w, None, x, oracle.MODE_BF16)      # bf16(sum) = 2^-8
    twice = oracle.bf16_encode(1.0 + float(_bf16_frac(s[0, 0])))
    assert twice == 0x3f80 and twice != good[0, 0]
