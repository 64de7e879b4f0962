"""Planted controls (CPU): results carrying a plausible kernel mistake must fail the checks
that the GPU parity tests apply to the kernels' results.

Each mistake is planted in a copy of the oracle's own output (or in the bytes the oracle
reads), never in GPU code: a top-k that breaks ties towards the higher id, a GEMV that skips
the last 16-row tile, a GEMV that drops one 32x32 block's E8M0 scale, a top-k whose per-chunk
lists hold k - 1 entries, and a top-k that ranks NaN first.
"""
import numpy as np
import pytest

import oracle
import synth
from parity import check_logits, check_topk, row_tol


def _tie_rows(V=700, seed=7):
    """Rows with exact ties straddling several k boundaries."""
    rng = np.random.default_rng(seed)
    rows = [rng.integers(-4, 5, V).astype(np.float32) / 4,   # coarse grid: many ties
            np.zeros(V, np.float32),                         # all equal
            rng.standard_normal(V).astype(np.float32)]
    rows[2][rng.choice(V, 40, replace=False)] = 8.0          # 40 tied winners
    return np.stack(rows)


def _topk_higher_id_ties(row, k):
    """A top-k that orders equal values by the higher id first (the planted mistake)."""
    e = [(float(v), i) for i, v in enumerate(row) if not np.isnan(v) and v != -np.inf]
    e.sort(key=lambda t: (-t[0], -t[1]))
    ids = [i for _, i in e[:k]] + [0] * max(0, k - len(e))
    vals = [row[i] for i in ids[:min(k, len(e))]] + [-np.inf] * max(0, k - len(e))
    return np.array(ids, np.int32), np.array(vals, np.float32)


@pytest.mark.parametrize("k", [1, 22, 31, 32, 33])
def test_control_ties_to_higher_id_fail(k):
    logits = _tie_rows()
    want_ids, want_vals = oracle.topk(logits, k)
    for r in range(logits.shape[0]):
        ids, vals = _topk_higher_id_ties(logits[r], k)
        # the GPU tests require the top-k of the GPU's own logits to equal the oracle's
        # bit for bit: this mistake must break that equality on every tie row
        assert not np.array_equal(ids, want_ids[r]), (r, k)


def test_control_skipped_last_tile_fails():
    V, H, R = 1000, 96, 3
    w = synth.random_head(V, H, seed=21, std=0.02)
    x = synth.random_acts(R, H, seed=22)
    good = oracle.gemv(oracle.FMT_BF16, w, None, x)
    bad = good.copy()
    last = (V - 1) // 16 * 16
    bad[:, last:] = 0.0                                      # the last tile never computed
    check_logits(good, good)
    with pytest.raises(AssertionError):
        check_logits(bad, good)


def test_control_dropped_block_scale_fails():
    V, H, R = 256, 128, 2
    w = synth.random_head(V, H, seed=31, std=0.02)
    x = synth.random_acts(R, H, seed=32)
    codes, scales = oracle.quant_block32(w)
    good = oracle.gemv(oracle.FMT_FP8_BLOCK32, codes, scales, x)
    dropped = scales.copy()
    dropped[3, 1] = 127                                      # one block read with scale 1.0
    bad = oracle.gemv(oracle.FMT_FP8_BLOCK32, codes, dropped, x)
    with pytest.raises(AssertionError):
        check_logits(bad, good)


def test_control_chunk_capacity_k_minus_1_fails():
    """A per-chunk list one entry short loses a winner when a chunk holds k of them."""
    V, k, chunk = 4096, 32, 2048
    rng = np.random.default_rng(41)
    row = rng.standard_normal(V).astype(np.float32)
    row[:k] = 4.0 + rng.random(k).astype(np.float32)         # every winner in chunk 0
    logits = row[None, :]
    tols = np.array([row_tol(row)])
    want_ids, want_vals = oracle.topk(logits, k)
    check_topk(want_ids, want_vals, logits, k, tols)
    # the planted pass 1 keeps k - 1 per chunk, so the merge sees only the chunks' lists
    kept = []
    for c in range(0, V, chunk):
        order = sorted(range(c, c + chunk), key=lambda i: (-row[i], i))
        kept += order[:k - 1]
    kept.sort(key=lambda i: (-row[i], i))
    ids = np.array([kept[:k]], np.int32)
    vals = row[ids]
    with pytest.raises(AssertionError):
        check_topk(ids, vals, logits, k, tols)


def test_control_nan_ranked_first_fails():
    V, k = 300, 8
    rng = np.random.default_rng(51)
    row = rng.standard_normal(V).astype(np.float32)
    row[[3, 77, 150]] = np.nan
    logits = row[None, :]
    tols = np.array([row_tol(row)])
    want_ids, want_vals = oracle.topk(logits, k)
    check_topk(want_ids, want_vals, logits, k, tols)
    # the planted mistake: NaN compares greater than every number (as an unguarded
    # float-to-integer key would order it)
    order = sorted(range(V), key=lambda i: (0 if np.isnan(row[i]) else 1, -np.nan_to_num(row[i]), i))
    ids = np.array([order[:k]], np.int32)
    vals = row[ids]
    with pytest.raises(AssertionError):
        check_topk(ids, vals, logits, k, tols)
