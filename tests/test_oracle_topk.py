"""Pins of the oracle's ordering, top-k, argmax and rescore (CPU).

Independent references: hand-worked cases of the pages' rules (tests/golden/topk_rules.json),
a brute-force Python sort with a (value descending, id ascending) key, exact rational
rescore dot products, and invariants (prefix property, argmax == top-1).
"""
from fractions import Fraction
import json
import os

import numpy as np
import pytest

import oracle
import synth
from fp_exact import rne_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_topk(row, k):
    elig = [(float(v), i) for i, v in enumerate(row) if not np.isnan(v) and v != -np.inf]
    elig.sort(key=lambda t: (-t[0], t[1]))
    ids = [i for _, i in elig[:k]] + [0] * max(0, k - len(elig))
    vals = [row[i] for i in ids[:len(elig[:k])]] + [-np.inf] * max(0, k - len(elig))
    return np.array(ids, np.int32), np.array(vals, np.float32)


def test_golden_rule_cases():
    g = json.load(open(os.path.join(GOLDEN, "topk_rules.json")))
    for case in g["cases"]:
        logits = np.array([[float(s) for s in case["logits"]]], np.float32)
        ids, vals = oracle.topk(logits, case["k"])
        want_vals = np.array([float(s) for s in case["vals"]], np.float32)
        assert list(ids[0]) == case["ids"], case["name"]
        assert np.array_equal(vals[0].view(np.uint32), want_vals.view(np.uint32)), case["name"]


def _planted_rows(V, rng):
    rows = [
        rng.standard_normal(V).astype(np.float32),
        (rng.integers(-3, 4, V) / 2).astype(np.float32),          # many exact ties
        np.full(V, np.nan, np.float32),
        np.full(V, -np.inf, np.float32),
        np.full(V, 1.5, np.float32),
        np.where(rng.random(V) < 0.5, np.float32(0.0), np.float32(-0.0)),
        (rng.integers(1, 4, V) * 1e-45).astype(np.float32),       # subnormals
        np.arange(V, dtype=np.float32),
        -np.arange(V, dtype=np.float32),
    ]
    mixed = rng.standard_normal(V).astype(np.float32)
    mixed[rng.random(V) < 0.2] = np.nan
    mixed[rng.random(V) < 0.1] = -np.inf
    mixed[rng.random(V) < 0.05] = np.inf
    rows.append(mixed)
    for m in (0, 1, 5, 21):
        r = np.full(V, -np.inf, np.float32)
        r[rng.choice(V, m, replace=False)] = rng.standard_normal(m).astype(np.float32)
        rows.append(r)
    ulp = np.float32(1.0)
    r = np.full(V, ulp, np.float32)
    r[::3] = np.nextafter(ulp, np.float32(2))
    r[1::3] = np.nextafter(ulp, np.float32(0))
    rows.append(r)
    return np.stack(rows)


@pytest.mark.parametrize("k", [1, 3, 22, 31, 32, 33, 64])
def test_topk_vs_brute_force(k):
    rng = np.random.default_rng(100 + k)
    logits = _planted_rows(70, rng)
    ids, vals = oracle.topk(logits, k)
    for r in range(logits.shape[0]):
        bi, bv = brute_topk(logits[r], k)
        assert np.array_equal(ids[r], bi), r
        assert np.array_equal(vals[r].view(np.uint32), bv.view(np.uint32)), r


def test_topk_prefix_and_argmax_invariants():
    rng = np.random.default_rng(7)
    logits = _planted_rows(200, rng)
    i512, v512 = oracle.topk(logits, 150)
    for k in (1, 2, 17, 64, 149):
        ik, vk = oracle.topk(logits, k)
        assert np.array_equal(ik, i512[:, :k]) and np.array_equal(vk.view(np.uint32), v512[:, :k].view(np.uint32))
    assert np.array_equal(oracle.argmax(logits), i512[:, 0])
    # eligible ids are distinct
    for r in range(logits.shape[0]):
        e = i512[r][v512[r] > -np.inf]
        assert len(set(e.tolist())) == len(e)


def test_beats_relation():
    assert oracle.beats(2.0, 5, 1.0, 0)
    assert oracle.beats(1.0, 0, 1.0, 5) and not oracle.beats(1.0, 5, 1.0, 0)
    assert oracle.beats(-0.0, 1, 0.0, 2) and not oracle.beats(0.0, 2, -0.0, 1)
    assert not oracle.beats(np.nan, 0, 1.0, 1) and oracle.beats(1.0, 1, np.nan, 0)
    assert not oracle.beats(-np.inf, 0, 1.0, 1) and oracle.beats(-1e30, 9, -np.inf, 0)
    assert oracle.beats(np.inf, 3, 1e38, 0)
    assert not oracle.beats(np.nan, 0, -np.inf, 1) and not oracle.beats(-np.inf, 1, np.nan, 0)


def _exact_rescore(wd, x, cand, use):
    wv = synth.bf16_bits_to_f32(wd)
    xv = synth.bf16_bits_to_f32(x)
    R, ck = cand.shape
    ex = np.empty((R, ck), np.float32)
    for r in range(R):
        for j in range(ck):
            c = int(cand[r, j])
            if use is not None and not use[r, j]:
                ex[r, j] = -np.inf
            elif c < 0 or c >= wd.shape[0]:
                ex[r, j] = np.nan
            else:
                ex[r, j] = rne_f32(sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xv[r], wv[c])), Fraction(0)))
    drafts = []
    for r in range(R):
        best = None
        for j in range(ck):
            e = ex[r, j]
            if np.isnan(e) or e == -np.inf:
                continue
            key = (-float(e), int(cand[r, j]))
            if best is None or key < best:
                best = key
        drafts.append(0 if best is None else best[1])
    return ex, np.array(drafts, np.int32)


def test_rescore_vs_exact_and_brute_argmax():
    V, H, R, ck = 60, 64, 3, 9
    wd = synth.random_head(V, H, 21)
    wd[10] = wd[11]                                  # duplicate rows: exact tie -> lower id
    x = synth.random_acts(R, H, 21)
    rng = np.random.default_rng(21)
    cand = rng.integers(0, V, (R, ck)).astype(np.int32)
    cand[0, :2] = [11, 10]
    cand[1, 3] = V + 5                               # out of range: NaN, never drafted
    cand[1, 4] = -1
    use = np.ones((R, ck), bool)
    use[2, 5:] = False                               # pads of a stage-1 list
    ex, d = oracle.rescore(wd, x, cand, use)
    ex2, d2 = _exact_rescore(wd, x, cand, use)
    assert np.array_equal(ex.view(np.uint32), ex2.view(np.uint32))
    assert np.array_equal(d, d2)
    # slot 0/1 tie exactly: the lower token id wins if they lead
    assert ex[0, 0] == ex[0, 1]


def test_rescore_no_eligible_candidate_drafts_zero():
    V, H = 8, 32
    wd = synth.random_head(V, H, 22)
    x = synth.random_acts(1, H, 22)
    x[0, 3] = 0x7FC0                                # NaN row: every exact logit NaN
    ex, d = oracle.rescore(wd, x, np.array([[5, 6, 7]], np.int32))
    assert np.all(np.isnan(ex)) and d[0] == 0
    ex, d = oracle.rescore(wd, synth.random_acts(1, H, 23), np.array([[5, 6]], np.int32),
                           np.zeros((1, 2), bool))
    assert np.all(ex == -np.inf) and d[0] == 0


def test_two_stage_draft_composition():
    V, H, R, k = 300, 64, 2, 16
    w = synth.random_head(V, H, 24, std=0.02)
    codes, s = oracle.quant_row(w)
    x = synth.random_acts(R, H, 24)
    out = oracle.draft(oracle.FMT_FP8_ROW, codes, s, x, k, dense_w=w)
    logits = oracle.gemv(oracle.FMT_FP8_ROW, codes, s, x)
    ids, vals = oracle.topk(logits, k)
    assert np.array_equal(out["ids"], ids)
    ex, d = _exact_rescore(w, x, ids, vals > -np.inf)
    assert np.array_equal(out["exact"].view(np.uint32), ex.view(np.uint32))
    assert np.array_equal(out["draft"], d)
    one = oracle.draft(oracle.FMT_FP8_ROW, codes, s, x, k)
    assert np.array_equal(one["draft"], ids[:, 0])
