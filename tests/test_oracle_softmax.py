"""Pins of the oracle's softmax statistics (CPU): O16, the top-k's probabilities and each row's
log-sum-exp, the reading of the top-1 "confidence" of "dsv41 Zig: the TFE draft head
(TF_DS_DRAFTER=eagle), off by default" (commit notes on the head's row kernels).

 * against scipy's logsumexp and softmax (library routines) on finite rows, and on rows with
   NaN and -inf removed first (they are not eligible);
 * closed forms: equal logits give 1/V and l + ln V; +inf entries share the mass equally and
   lse is +inf; no eligible logit gives lse = -inf and zero probabilities;
 * shift invariance: adding c to a row leaves the probabilities and moves lse by c (exactly
   representable values);
 * a planted mistake: a softmax that keeps -inf / NaN entries in the sum (as a plain
   float sum would propagate NaN) fails.
"""
import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle


def test_softmax_matches_scipy():
    rng = np.random.default_rng(1)
    R, V, k = 6, 3000, 64
    logits = (rng.standard_normal((R, V)) * 3).astype(np.float32)
    logits[3, ::7] = np.nan
    logits[4, ::5] = -np.inf
    ids, vals, probs, lse = oracle.topk_softmax(logits, k)
    for r in range(R):
        row = logits[r].astype(np.float64)
        el = row[~np.isnan(row) & (row != -np.inf)]
        want_lse = logsumexp(el)
        assert abs(float(lse[r]) - want_lse) <= 1e-6 * max(1.0, abs(want_lse))
        p = softmax(el)
        full = np.zeros(V)
        full[~np.isnan(row) & (row != -np.inf)] = p
        np.testing.assert_allclose(probs[r], full[ids[r]], rtol=1e-6, atol=0)


@pytest.mark.parametrize("V", [1, 7, 5000])
def test_equal_logits(V):
    logits = np.full((1, V), 2.5, np.float32)
    k = min(V, 8)
    _, _, probs, lse = oracle.topk_softmax(logits, k)
    np.testing.assert_allclose(probs[0], np.full(k, 1.0 / V), rtol=1e-7)
    assert abs(float(lse[0]) - (2.5 + np.log(V))) <= 1e-6


def test_infinities_and_empty_rows():
    inf, nan = np.inf, np.nan
    logits = np.array([[1.0, inf, 3.0, inf, inf],
                       [nan, -inf, nan, -inf, nan],
                       [-inf, 5.0, nan, -inf, -inf]], np.float32)
    ids, vals, probs, lse = oracle.topk_softmax(logits, 4)
    assert np.array_equal(ids[0, :3], [1, 3, 4])
    np.testing.assert_allclose(probs[0], [1 / 3, 1 / 3, 1 / 3, 0.0], rtol=1e-7)
    assert lse[0] == inf
    assert lse[1] == -inf and not probs[1].any()
    assert probs[2, 0] == 1.0 and lse[2] == 5.0 and not probs[2, 1:].any()


def test_shift_invariance():
    rng = np.random.default_rng(2)
    base = (rng.integers(-64, 64, (3, 500)) / 8).astype(np.float32)   # exact under the shift
    _, _, p0, l0 = oracle.topk_softmax(base, 32)
    _, _, p1, l1 = oracle.topk_softmax(base + np.float32(16), 32)
    np.testing.assert_allclose(p1, p0, rtol=1e-6)
    np.testing.assert_allclose(l1, l0 + 16, rtol=0, atol=1e-5)


def test_control_ineligible_in_sum_fails():
    row = np.array([[1.0, np.nan, 2.0, -np.inf]], np.float32)
    _, vals, probs, lse = oracle.topk_softmax(row, 2)
    with np.errstate(invalid="ignore"):
        planted = float(np.log(np.sum(np.exp(row.astype(np.float64)))))   # NaN propagates
    assert not np.isfinite(planted) and np.isfinite(lse[0])
