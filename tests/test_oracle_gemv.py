"""Pins of the oracle's GEMV (O5) in all three head formats (CPU).

Independent references: exact rational dot products rounded to float32 by a hand-written
RNE (tests/fp_exact.py), numpy's float64 matmul, torch's FP8 decoders for dequantization,
and closed forms (identity / permutation / equal-row heads, zero and NaN activations,
scale doubling).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from fp_exact import e4m3_table_torch, e8m0_table_torch, rne_f32


def _wvals_bf16(w):
    return synth.bf16_bits_to_f32(w).astype(np.float64)


def _wvals_block(codes, scales):
    V, H = codes.shape
    e = e8m0_table_torch()[scales].astype(np.float64)
    return e4m3_table_torch()[codes].astype(np.float64) * np.repeat(np.repeat(e, 32, 0), 32, 1)[:V, :H]


def _wvals_row(codes, s):
    return e4m3_table_torch()[codes].astype(np.float64) * s.astype(np.float64)[:, None]


def _exact_logits(wv, xv):
    """float32 RNE of the exact rational sum, for every (r, v)."""
    R, V = xv.shape[0], wv.shape[0]
    out = np.empty((R, V), np.float32)
    for r in range(R):
        xr = [Fraction(float(a)) for a in xv[r]]
        for v in range(V):
            out[r, v] = rne_f32(sum((xr[h] * Fraction(float(wv[v, h])) for h in range(wv.shape[1])), Fraction(0)))
    return out


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_bf16_gemv_equals_exact_rational(seed):
    V, H, R = 24, 64, 3
    w = synth.random_head(V, H, seed)
    x = synth.random_acts(R, H, seed)
    got = oracle.gemv(oracle.FMT_BF16, w, None, x)
    want = _exact_logits(_wvals_bf16(w), synth.bf16_bits_to_f32(x))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("seed", [4, 5])
def test_fp8_block_gemv_equals_exact_rational(seed):
    V, H, R = 40, 64, 2
    w = synth.random_head(V, H, seed, std=0.02)
    codes, scales = oracle.quant_block32(w)
    x = synth.random_acts(R, H, seed)
    got = oracle.gemv(oracle.FMT_FP8_BLOCK32, codes, scales, x)
    want = _exact_logits(_wvals_block(codes, scales), synth.bf16_bits_to_f32(x))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_fp8_row_gemv_equals_exact_rational():
    V, H, R = 20, 64, 2
    w = synth.random_head(V, H, 6, std=0.02)
    codes, s = oracle.quant_row(w)
    x = synth.random_acts(R, H, 6)
    got = oracle.gemv(oracle.FMT_FP8_ROW, codes, s, x)
    want = _exact_logits(_wvals_row(codes, s), synth.bf16_bits_to_f32(x))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("fmt", ["bf16", "block", "row"])
def test_gemv_vs_numpy_float64(fmt):
    V, H, R = 300, 512, 5
    w = synth.random_head(V, H, 11, std=0.02)
    x = synth.random_acts(R, H, 11)
    if fmt == "bf16":
        got = oracle.gemv(oracle.FMT_BF16, w, None, x)
        wv = _wvals_bf16(w)
    elif fmt == "block":
        c, s = oracle.quant_block32(w)
        got = oracle.gemv(oracle.FMT_FP8_BLOCK32, c, s, x)
        wv = _wvals_block(c, s)
    else:
        c, s = oracle.quant_row(w)
        got = oracle.gemv(oracle.FMT_FP8_ROW, c, s, x)
        wv = _wvals_row(c, s)
    ref = synth.bf16_bits_to_f32(x).astype(np.float64) @ wv.T
    assert np.allclose(got, ref, rtol=2e-7, atol=1e-9 * np.abs(ref).max())


def test_sampled_rows_equal_full():
    V, H, R = 97, 96, 4
    w = synth.random_head(V, H, 12, std=0.02)
    c, s = oracle.quant_block32(w)
    x = synth.random_acts(R, H, 12)
    full = oracle.gemv(oracle.FMT_FP8_BLOCK32, c, s, x)
    vids = np.array([96, 0, 31, 32, 50, 50])
    part = oracle.gemv(oracle.FMT_FP8_BLOCK32, c, s, x, vids)
    assert np.array_equal(part, full[:, vids])


def test_cross_format_block_equals_bf16_of_dequant():
    """FP8 block head == bf16 head holding the dequantized values, bit for bit: the
    dequantized weights are exact in bf16 and both sums are the same reals in the same
    order.  The dequantization here uses torch's decoders, not the oracle's."""
    V, H, R = 96, 256, 3
    w = synth.random_head(V, H, 13, std=0.02)
    c, s = oracle.quant_block32(w)
    deq = _wvals_block(c, s).astype(np.float32)
    wb = synth.to_bf16_bits(deq)
    assert np.array_equal(synth.bf16_bits_to_f32(wb), deq)   # exact in bf16
    x = synth.random_acts(R, H, 13)
    a = oracle.gemv(oracle.FMT_FP8_BLOCK32, c, s, x)
    b = oracle.gemv(oracle.FMT_BF16, wb, None, x)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_identity_and_permutation_heads():
    H = 64
    x = synth.random_acts(2, H, 14)
    codes = np.zeros((H, H), np.uint8)
    codes[np.arange(H), np.arange(H)] = 0x38            # 1.0
    scales = np.full((2, 2), 127, np.uint8)              # 2^0
    got = oracle.gemv(oracle.FMT_FP8_BLOCK32, codes, scales, x)
    assert np.array_equal(got, synth.bf16_bits_to_f32(x))
    perm = np.random.default_rng(0).permutation(H)
    wp = np.zeros((H, H), np.uint16)
    wp[np.arange(H), perm] = 0x3F80                      # bf16 1.0
    got = oracle.gemv(oracle.FMT_BF16, wp, None, x)
    assert np.array_equal(got, synth.bf16_bits_to_f32(x)[:, perm])
    s = np.full(H, 0.5, np.float32)
    got = oracle.gemv(oracle.FMT_FP8_ROW, codes, s, x)
    assert np.array_equal(got, synth.bf16_bits_to_f32(x) * np.float32(0.5))


def test_scale_byte_doubles_block_contribution():
    """Raising one E8M0 byte by one doubles exactly that block's share of each logit.
    Small integers keep every sum exact, so the difference is checked exactly."""
    V, H = 64, 64
    rng = np.random.default_rng(15)
    codes = np.array([0x38, 0x40, 0xB8, 0x00, 0x30], np.uint8)[rng.integers(0, 5, (V, H))]
    scales = np.full((2, 2), 127, np.uint8)
    x = synth.to_bf16_bits(rng.integers(-3, 4, (2, H)).astype(np.float32))
    base = oracle.gemv(oracle.FMT_FP8_BLOCK32, codes, scales, x).astype(np.float64)
    scales2 = scales.copy()
    scales2[1, 0] = 128
    got = oracle.gemv(oracle.FMT_FP8_BLOCK32, codes, scales2, x).astype(np.float64)
    xv = synth.bf16_bits_to_f32(x).astype(np.float64)
    share = xv[:, :32] @ e4m3_table_torch()[codes[32:, :32]].astype(np.float64).T
    assert np.array_equal(got[:, :32], base[:, :32])
    assert np.array_equal(got[:, 32:] - base[:, 32:], share)


def test_zero_and_nan_activation_rows():
    V, H = 50, 64
    w = synth.random_head(V, H, 16, std=0.02)
    x = synth.random_acts(3, H, 16)
    x[0] = 0
    x[1, 7] = 0x7FC0                                     # NaN
    x[2, 9] = 0x7F80                                     # +inf
    got = oracle.gemv(oracle.FMT_BF16, w, None, x)
    assert np.all(got[0] == 0)
    assert np.all(np.isnan(got[1]))
    wcol = synth.bf16_bits_to_f32(w)[:, 9]
    assert np.array_equal(np.isposinf(got[2]), wcol > 0)
    assert np.array_equal(np.isneginf(got[2]), wcol < 0)
    assert np.array_equal(np.isnan(got[2]), wcol == 0)
