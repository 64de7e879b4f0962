"""Pins of the oracle's number formats and quantizers (CPU).

Independent references: torch's bfloat16 / float8_e4m3fn / float8_e8m0fnu dtypes (library
decoders and an RNE encoder), a brute-force nearest-code search, and closed-form facts the
pages fix (the per-row rule s = amax/448 maps the row's largest magnitude to the largest
E4M3 code; 32x32 blocks with E8M0 scales).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from fp_exact import brute_e4m3_encode, e4m3_table_torch, e8m0_table_torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_decode_all_patterns_vs_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    got = np.array([oracle.bf16_value(b) for b in bits[::97]] +
                   [oracle.bf16_value(b) for b in (0x7F80, 0xFF80, 0x7FC0, 0x8000, 0x0001)])
    want = np.concatenate([ref[::97], ref[[0x7F80, 0xFF80, 0x7FC0, 0x8000, 0x0001]]])
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok].astype(np.float64))
    assert np.signbit(got[-2])          # -0 keeps its sign


def test_e4m3_decode_all_codes_vs_torch():
    table = e4m3_table_torch()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan = np.isnan(table)
    assert np.array_equal(np.isnan(got), nan)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(got[~nan], table[~nan].astype(np.float64))


def test_e4m3_golden_points():
    """Facts the pages fix: the largest finite magnitude is the per-row rule's divisor."""
    g = json.load(open(os.path.join(GOLDEN, "fp8_facts.json")))
    assert oracle.e4m3_value(g["e4m3_max_code"]) == g["e4m3_max"]
    assert max(abs(oracle.e4m3_value(c)) for c in range(256)
               if not np.isnan(oracle.e4m3_value(c))) == g["e4m3_max"]
    for code, val in g["e4m3_points"]:
        assert oracle.e4m3_value(int(code, 16)) == val


def test_e8m0_decode_all_bytes_vs_torch():
    table = e8m0_table_torch()
    got = np.array([oracle.e8m0_value(b) for b in range(256)])
    assert np.isnan(got[255]) and np.isnan(table[255])
    assert np.array_equal(got[:255], table[:255].astype(np.float64))


def _sweep_values():
    """Every E4M3 value, every midpoint between neighbours (the ties), points just either
    side of each midpoint, beyond-range values and zeros."""
    table = e4m3_table_torch()
    pos = np.unique(table[:0x7F].astype(np.float64))
    mids = (pos[1:] + pos[:-1]) / 2
    vals = [pos, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
            np.nextafter(mids.astype(np.float32), np.float32(1e9)),
            np.array([448.0, 449.0, 463.99, 464.0, 465.0, 1e6, 3.0e38, 2.0 ** -10,
                      2.0 ** -11, 1e-30, 0.0])]
    v = np.concatenate([a.astype(np.float32) for a in vals])
    return np.concatenate([v, -v])


def test_e4m3_encode_vs_brute_force():
    table = e4m3_table_torch()
    for f in _sweep_values():
        assert oracle.e4m3_encode(f) == brute_e4m3_encode(f, table), f


def test_e4m3_encode_vs_torch_cast_in_range():
    rng = np.random.default_rng(7)
    f = np.concatenate([rng.standard_normal(20000).astype(np.float32) * s
                        for s in (1e-3, 0.05, 1.0, 30.0, 150.0)])
    f = np.concatenate([f[np.abs(f) <= 448], _sweep_values()])
    f = f[np.abs(f) <= 448]
    ref = torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(v) for v in f], np.uint8)
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates_and_roundtrips():
    assert oracle.e4m3_encode(1e30) == 0x7E and oracle.e4m3_encode(-1e30) == 0xFE
    assert oracle.e4m3_encode(np.inf) == 0x7E
    assert oracle.e4m3_encode(np.nan) & 0x7F == 0x7F
    for c in range(256):
        v = oracle.e4m3_value(c)
        if not np.isnan(v):
            assert oracle.e4m3_encode(v) == c


def _dequant_row(codes, scale):
    return e4m3_table_torch()[codes].astype(np.float64) * scale.astype(np.float64)[:, None]


def test_quant_row_rule():
    """Q1: s = float(amax/448) (a float32 division), codes = RNE(w/s)."""
    w = synth.random_head(40, 96, seed=3, std=0.02)
    w[5] = 0                                      # an all-zero row
    w[7, :] = synth.to_bf16_bits(np.full(96, -3.5, np.float32))   # a constant row
    codes, s = oracle.quant_row(w)
    wf = synth.bf16_bits_to_f32(w)
    amax = np.abs(wf).max(axis=1)
    assert np.array_equal(s, (amax / np.float32(448)).astype(np.float32))
    assert s[5] == 0 and not codes[5].any()
    nz = amax > 0
    # the row's largest magnitude maps to +-448 exactly
    for v in np.nonzero(nz)[0]:
        h = int(np.argmax(np.abs(wf[v])))
        assert codes[v, h] & 0x7F == 0x7E
    q = (wf[nz] / s[nz, None]).astype(np.float32)
    ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes[nz], ref)
    # error bound: half a quantum of the E4M3 grid at |q| times s
    deq = _dequant_row(codes, s)
    qa = np.abs(q.astype(np.float64))
    quantum = np.where(qa < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(qa, 1e-30))) - 3))
    assert np.all(np.abs(deq[nz] - wf[nz]) <= 0.5 * quantum * s[nz, None].astype(np.float64) * (1 + 1e-6))


def _dequant_block(codes, scales):
    e = e8m0_table_torch()[scales].astype(np.float64)
    V, H = codes.shape
    full = np.repeat(np.repeat(e, 32, axis=0), 32, axis=1)[:V, :H]
    return e4m3_table_torch()[codes].astype(np.float64) * full


@pytest.mark.parametrize("V", [64, 70])
def test_quant_block32_rule(V):
    """Q2: e is the least integer with amax <= 448*2^e; codes = RNE(w * 2^-e)."""
    H = 128
    w = synth.random_head(V, H, seed=V, std=0.02)
    w[32:64, 32:64] = 0                              # an all-zero block
    w[0:32, 64:96] = synth.to_bf16_bits(np.full((32, 32), 448.0 * 2 ** -5, np.float32))  # amax exactly on 448*2^e
    codes, scales = oracle.quant_block32(w)
    assert scales.shape == ((V + 31) // 32, H // 32)
    wf = synth.bf16_bits_to_f32(w).astype(np.float64)
    for bv in range(scales.shape[0]):
        for bh in range(scales.shape[1]):
            blk = wf[bv * 32:bv * 32 + 32, bh * 32:bh * 32 + 32]
            amax = np.abs(blk).max()
            e = int(scales[bv, bh]) - 127
            if amax == 0:
                assert scales[bv, bh] == 127
                continue
            assert amax <= 448.0 * 2.0 ** e and amax > 448.0 * 2.0 ** (e - 1)
            cb = codes[bv * 32:bv * 32 + 32, bh * 32:bh * 32 + 32]
            mags = e4m3_table_torch()[cb & 0x7F]
            assert mags.max() >= 224 and mags.max() <= 448
    assert scales[0, 2] == 127 - 5
    deq = _dequant_block(codes, scales)
    q = np.ldexp(wf, -(np.repeat(np.repeat(scales.astype(np.int64) - 127, 32, 0), 32, 1)[:V, :H]))
    ref = torch.from_numpy(q.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    assert np.all(np.abs(deq - wf) <= np.abs(wf) * 2 ** -4 + 2.0 ** -9 * 2.0 ** (scales.astype(np.float64).max() - 127))


def test_quant_block32_partial_last_block():
    w = synth.random_head(33, 64, seed=9, std=1.0)
    codes, scales = oracle.quant_block32(w)
    assert scales.shape == (2, 2)
    # the partial block is scaled by its one existing row only
    amax = np.abs(synth.bf16_bits_to_f32(w[32])).reshape(2, 32).max(axis=1)
    for bh in range(2):
        e = int(scales[1, bh]) - 127
        assert amax[bh] <= 448 * 2.0 ** e and amax[bh] > 448 * 2.0 ** (e - 1)
