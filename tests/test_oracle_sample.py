"""Pins of the oracle's keyed sampler (CPU): O17 and its generator, from "DeepSeek-V4.1:
performance hooks and host checks", commit notes on the serving module's sampler (a pick
keyed by seed, position and token id; candidates and nucleus statistics).  The pages give no
formula; what is pinned is the reading (Gumbel-max over the nucleus / min-p survivors, the
uniforms from Philox4x64-10).

 * Philox4x64-10 against numpy's Philox bit generator (the same published generator; numpy
   increments its counter before each block, so its counter c yields block c + 1);
 * the pick's law: over many seeds the frequencies of the picks follow q_j / sum of the kept
   q (a chi-square test at p > 1e-4), for a temperature, a nucleus and a min-p case;
 * limits: temperature 0 and top_p -> 0 pick the first candidate, min_p = 1 keeps only the
   entries tied with the first; pads are never picked; a row of pads gives token 0;
 * the key: the same (seed, position) picks the same token when the list is shuffled (the
   keyed uniforms go with the token ids), and different positions or seeds pick differently;
 * a planted mistake: keying the uniforms by list slot instead of token id fails the shuffle
   invariance.
"""
import numpy as np
import pytest
from scipy.stats import chisquare

import oracle


def test_philox_matches_numpy():
    rng = np.random.default_rng(5)
    for _ in range(20):
        ctr = rng.integers(1, 2**63, 4, dtype=np.uint64)
        key = rng.integers(0, 2**63, 2, dtype=np.uint64)
        ref = np.random.Philox(counter=[int(ctr[0]) - 1, int(ctr[1]), int(ctr[2]), int(ctr[3])],
                               key=[int(key[0]), int(key[1])]).random_raw(4)
        assert np.array_equal(oracle.philox4x64(ctr, key), np.asarray(ref, np.uint64))


def test_keyed_uniform_range_and_mean():
    u = np.array([oracle.keyed_uniform(7, p, i) for p in range(50) for i in range(200)])
    assert np.all((u > 0) & (u < 1))
    assert abs(u.mean() - 0.5) < 0.01 and abs(u.var() - 1 / 12) < 0.005


def _law(vals, T, top_p, min_p):
    v = np.asarray(vals, np.float64)
    el = v > -np.inf
    q = np.where(el, np.exp((v - v[0]) / T), 0.0)
    before = np.concatenate([[0.0], np.cumsum(q)[:-1]])
    keep = el & ((np.arange(v.size) == 0) | ((before < top_p * q.sum()) & (q >= min_p)))
    return np.where(keep, q, 0.0) / np.where(keep, q, 0.0).sum()


@pytest.mark.parametrize("T,top_p,min_p", [(1.0, 1.0, 0.0), (0.7, 0.8, 0.0), (1.3, 1.0, 0.05)])
def test_pick_law(T, top_p, min_p):
    vals = np.array([[2.0, 1.6, 1.5, 0.9, 0.3, -0.4, -1.0, -np.inf]], np.float32)
    ids = np.array([[40, 7, 19, 3, 88, 51, 12, 0]], np.int32)
    N = 6000
    picks = np.empty(N, np.int32)
    for s in range(N):
        picks[s] = oracle.sample(ids, vals, T, top_p, min_p, seed=1000 + s, pos=[17])[0][0]
    p = _law(vals[0], T, top_p, min_p)
    kept = p > 0
    counts = np.array([np.sum(picks == i) for i in ids[0]])
    assert counts[~kept].sum() == 0
    stat, pval = chisquare(counts[kept], N * p[kept])
    assert pval > 1e-4, (counts, N * p)


def test_limits():
    vals = np.array([[3.0, 3.0, 2.0, 1.0],
                     [1.0, 0.5, -np.inf, -np.inf],
                     [-np.inf, -np.inf, -np.inf, -np.inf]], np.float32)
    ids = np.array([[9, 4, 5, 6], [2, 8, 0, 0], [0, 0, 0, 0]], np.int32)
    pos = [3, 4, 5]
    t, kept, _ = oracle.sample(ids, vals, 0.0, 1.0, 0.0, 11, pos)
    assert list(t) == [9, 2, 0] and list(kept) == [1, 1, 0]
    t, kept, _ = oracle.sample(ids, vals, 1.0, 1e-9, 0.0, 11, pos)
    assert list(t) == [9, 2, 0] and list(kept) == [1, 1, 0]
    t, kept, _ = oracle.sample(ids, vals, 1.0, 1.0, 1.0, 11, pos)
    assert t[0] in (9, 4) and kept[0] == 2 and t[1] == 2 and kept[1] == 1
    for s in range(200):
        t, kept, _ = oracle.sample(ids, vals, 5.0, 1.0, 0.0, s, pos)
        assert t[1] in (2, 8) and kept[1] == 2 and t[2] == 0


def test_keyed_by_token_id():
    rng = np.random.default_rng(9)
    vals = np.sort(rng.standard_normal(64).astype(np.float32))[::-1].copy()[None]
    ids = rng.choice(100000, 64, replace=False).astype(np.int32)[None]
    base = [oracle.sample(ids, vals, 1.0, 1.0, 0.0, s, [123])[0][0] for s in range(40)]
    # shuffle the list; with top_p = 1 and min_p = 0 every candidate is kept whatever the
    # order, and the largest value goes back to slot 0 (v_0 only shifts every score alike)
    perm = rng.permutation(64)
    sv, si = vals[:, perm], ids[:, perm]
    first = int(np.argmax(sv[0]))
    sv[0, [0, first]] = sv[0, [first, 0]]
    si[0, [0, first]] = si[0, [first, 0]]
    shuf = [oracle.sample(si, sv, 1.0, 1.0, 0.0, s, [123])[0][0] for s in range(40)]
    assert base == shuf
    other = [oracle.sample(ids, vals, 1.0, 1.0, 0.0, s, [124])[0][0] for s in range(40)]
    assert base != other
    # planted mistake: uniforms keyed by list slot instead of token id
    def slot_keyed(iv, vv, seed):
        v = vv[0].astype(np.float64)
        sc = [(v[j] - v[0]) - np.log(-np.log(oracle.keyed_uniform(seed, 123, j))) for j in range(64)]
        return iv[0][int(np.argmax(sc))]
    a = [slot_keyed(ids, vals, s) for s in range(40)]
    b = [slot_keyed(si, sv, s) for s in range(40)]
    assert a != b
