"""Pins of the oracle's draft-vocabulary subset head (CPU).

O12 (the subset head: row j is row ids[j] of the head, with its row scale) and O13 (the top-k
of a subset head's logits, whose column j is token idmap[j]), from "nemotron: Super's MTP
drafts on the draft vocabulary's FP8 rows while a stream's text is covered, same replies",
'What this changes'.  Each is pinned to something other than itself:

 * O12 against numpy's fancy indexing (rows and row scales), and through O5: the subset
   head's logits are the full head's logits at the subset's ids, bit for bit (O5's own
   column-subset form, pinned in test_oracle_gemv.py), so a row or scale taken from the
   wrong id fails;
 * O13 against a brute-force sort of (logit, token id) pairs written here, with maps that
   are not increasing (so the tie rule by token id is exercised apart from the tie rule by
   column), and the reduction to O8 for an increasing map;
 * planted mistakes: a map applied to the pads, and ties resolved by column under a
   decreasing map, must fail these checks.
"""
import numpy as np
import pytest

import oracle
import synth


def _brute_topk_tokens(row, idmap, k):
    e = [(float(v), int(idmap[j])) for j, v in enumerate(row)
         if not np.isnan(v) and v != -np.inf]
    e.sort(key=lambda t: (-t[0], t[1]))
    ids = [t for _, t in e[:k]] + [0] * max(0, k - len(e))
    vals = [v for v, _ in e[:k]] + [-np.inf] * max(0, k - len(e))
    return np.array(ids, np.int32), np.array(vals, np.float32)


@pytest.mark.parametrize("fmt", [oracle.FMT_BF16, oracle.FMT_FP8_ROW])
def test_subset_rows_are_indexed_rows(fmt):
    V, H = 300, 64
    w = synth.random_head(V, H, seed=61, std=0.02)
    if fmt == oracle.FMT_FP8_ROW:
        w, scale = oracle.quant_row(w)
    else:
        scale = None
    ids = np.array([299, 0, 17, 17, 150, -1, 300, 5, 2**31 - 1], np.int32)
    sw, ss = oracle.subset_rows(fmt, w, scale, ids)
    ok = (ids >= 0) & (ids < V)
    assert np.array_equal(sw[ok], w[ids[ok]])
    assert not sw[~ok].any()
    if scale is None:
        assert ss is None
    else:
        assert np.array_equal(ss[ok], scale[ids[ok]])
        assert np.all(ss[~ok] == 0)


def test_subset_rows_refuse_block_scales():
    w = synth.random_head(64, 64, seed=62, std=0.02)
    codes, scales = oracle.quant_block32(w)
    with pytest.raises(ValueError):
        oracle.subset_rows(oracle.FMT_FP8_BLOCK32, codes, scales, np.arange(4, dtype=np.int32))


@pytest.mark.parametrize("fmt", [oracle.FMT_BF16, oracle.FMT_FP8_ROW])
def test_subset_logits_are_full_logits_at_ids(fmt):
    V, H, R = 1000, 96, 3
    w = synth.random_head(V, H, seed=63, std=0.02)
    scale = None
    if fmt == oracle.FMT_FP8_ROW:
        w, scale = oracle.quant_row(w)
    x = synth.random_acts(R, H, seed=64)
    ids = synth.token_ids(V, 371, seed=65)
    sw, ss = oracle.subset_rows(fmt, w, scale, ids)
    sub = oracle.gemv(fmt, sw, ss, x)
    full_at = oracle.gemv(fmt, w, scale, x, vids=ids)
    assert np.array_equal(sub.view(np.uint32), full_at.view(np.uint32))


def test_subset_wrong_scale_index_fails():
    """A gather that takes each row's scale from the next id must change the logits."""
    V, H, R = 500, 64, 2
    w = synth.random_head(V, H, seed=66, std=0.02)
    codes, scale = oracle.quant_row(w)
    x = synth.random_acts(R, H, seed=67)
    ids = synth.token_ids(V, 100, seed=68)
    sw, ss = oracle.subset_rows(oracle.FMT_FP8_ROW, codes, scale, ids)
    bad = scale[np.minimum(ids + 1, V - 1)]
    want = oracle.gemv(oracle.FMT_FP8_ROW, codes, scale, x, vids=ids)
    got = oracle.gemv(oracle.FMT_FP8_ROW, sw, bad, x)
    assert not np.array_equal(got, want)


@pytest.mark.parametrize("order", ["increasing", "decreasing", "shuffled"])
@pytest.mark.parametrize("k", [1, 5, 40, 64])
def test_topk_mapped_brute_force(order, k):
    rng = np.random.default_rng(69)
    n, V = 50, 10000
    idmap = synth.token_ids(V, n, seed=70)
    if order == "decreasing":
        idmap = idmap[::-1].copy()
    elif order == "shuffled":
        idmap = rng.permutation(idmap).astype(np.int32)
    rows = np.stack([rng.integers(-3, 4, n).astype(np.float32) / 2,        # many ties
                     rng.standard_normal(n).astype(np.float32),
                     np.full(n, np.nan, np.float32)])
    rows[1, [4, 9]] = [np.nan, -np.inf]
    ids, vals = oracle.topk_mapped(rows, k, idmap)
    for r in range(rows.shape[0]):
        bi, bv = _brute_topk_tokens(rows[r], idmap, k)
        assert np.array_equal(ids[r], bi), (order, k, r)
        assert np.array_equal(vals[r].view(np.uint32), bv.view(np.uint32))


def test_topk_mapped_increasing_is_mapped_topk():
    rng = np.random.default_rng(71)
    n = 2000
    idmap = synth.token_ids(131072, n, seed=72)
    rows = rng.integers(-6, 7, size=(4, n)).astype(np.float32) / 4
    rows[3, :1990] = -np.inf                                    # fewer eligible than k
    k = 33
    ids, vals = oracle.topk_mapped(rows, k, idmap)
    li, lv = oracle.topk(rows, k)
    real = lv > -np.inf
    assert np.array_equal(vals.view(np.uint32), lv.view(np.uint32))
    assert np.array_equal(ids[real], idmap[li[real]])
    assert np.all(ids[~real] == 0)


def test_control_map_applied_to_pads_fails():
    n = 20
    idmap = np.arange(100, 100 + n, dtype=np.int32)
    row = np.full((1, n), -np.inf, np.float32)
    row[0, :3] = [1.0, 2.0, 3.0]
    ids, _ = oracle.topk_mapped(row, 8, idmap)
    li, lv = oracle.topk(row, 8)
    planted = idmap[li]                                          # pads mapped to idmap[0]
    assert not np.array_equal(planted, ids)


def test_control_column_ties_under_decreasing_map_fail():
    n = 12
    idmap = np.arange(1000, 1000 - n, -1, dtype=np.int32)       # decreasing token ids
    row = np.zeros((1, n), np.float32)                           # all tied
    ids, _ = oracle.topk_mapped(row, 4, idmap)
    li, _ = oracle.topk(row, 4)
    assert not np.array_equal(idmap[li], ids)                    # column ties != token ties
    assert np.array_equal(ids[0], np.sort(idmap)[:4])
