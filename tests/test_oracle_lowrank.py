"""Pins of the oracle's low-rank stage 1 (CPU): O15 = O14 (bf16 rank-r activations) then O5
then O8 (and O10), from "dsv41 Zig: the TFE draft head (TF_DS_DRAFTER=eagle), off by
default", two_stage commit note.

 * an identity `down` (rank = H) makes t = x exactly, so the low-rank logits equal O5 of `up`
   on x bit for bit;
 * a permutation `down` (row j = unit vector p(j)) makes t[j] = x[p(j)], so the logits equal
   O5 of the head whose column p(j) is up's column j, and a transposed square permutation
   (t = x P instead of x P^T) gives other logits;
 * a dense `down` on small inputs: t equals exact rational arithmetic rounded to bf16 (via
   O14's own pin), and the conditional form with a given t reproduces the logits of that t.
"""
import numpy as np

import oracle
import synth

ONE = np.uint16(0x3f80)


def test_identity_down_gives_plain_logits():
    H, V, R, k = 64, 300, 3, 10
    down = np.zeros((H, H), np.uint16)
    down[np.arange(H), np.arange(H)] = ONE
    up = synth.random_head(V, H, seed=1, std=0.05)
    x = synth.random_acts(R, H, seed=2)
    o = oracle.draft_lowrank((oracle.FMT_BF16, down, None), (oracle.FMT_BF16, up, None), x, k)
    assert np.array_equal(o["t"], x)
    plain = oracle.gemv(oracle.FMT_BF16, up, None, x)
    assert np.array_equal(o["logits"].view(np.uint32), plain.view(np.uint32))
    ids, vals = oracle.topk(plain, k)
    assert np.array_equal(o["ids"], ids) and np.array_equal(o["draft"], ids[:, 0])


def test_permutation_down_fixes_orientation():
    H, rk, V, R = 96, 32, 200, 2
    rng = np.random.default_rng(3)
    p = rng.choice(H, rk, replace=False)              # t[j] = x[p[j]]
    down = np.zeros((rk, H), np.uint16)
    down[np.arange(rk), p] = ONE
    up = synth.random_head(V, rk, seed=4, std=0.05)
    x = synth.random_acts(R, H, seed=5)
    o = oracle.draft_lowrank((oracle.FMT_BF16, down, None), (oracle.FMT_BF16, up, None), x, 4)
    assert np.array_equal(o["t"], x[:, p])
    wide = np.zeros((V, H), np.uint16)                # up's column j at column p[j]
    wide[:, p] = up
    want = oracle.gemv(oracle.FMT_BF16, wide, None, x)
    assert np.array_equal(o["logits"].view(np.uint32), want.view(np.uint32))


def test_control_transposed_down_fails():
    """With a square permutation down = P (t = x P^T), a transposed down (t = x P) takes
    x[p^-1(j)] instead of x[p(j)]: the logits must differ."""
    H, V, R = 64, 150, 2
    rng = np.random.default_rng(10)
    p = rng.permutation(H)
    assert np.any(p[p] != np.arange(H))               # not an involution
    P = np.zeros((H, H), np.uint16)
    P[np.arange(H), p] = ONE
    up = synth.random_head(V, H, seed=11, std=0.05)
    x = synth.random_acts(R, H, seed=12)
    good = oracle.draft_lowrank((oracle.FMT_BF16, P, None), (oracle.FMT_BF16, up, None), x, 4)
    bad = oracle.draft_lowrank((oracle.FMT_BF16, np.ascontiguousarray(P.T), None),
                               (oracle.FMT_BF16, up, None), x, 4)
    assert np.array_equal(good["t"], x[:, p])
    assert not np.array_equal(bad["logits"], good["logits"])


def test_dense_down_and_conditional_form():
    H, rk, V, R, k = 128, 64, 500, 3, 16
    down = synth.random_head(rk, H, seed=6, std=1 / np.sqrt(H))
    up = synth.random_head(V, rk, seed=7, std=0.05)
    x = synth.random_acts(R, H, seed=8)
    dense = synth.random_head(V, H, seed=9, std=0.02)
    dn, u = (oracle.FMT_BF16, down, None), (oracle.FMT_BF16, up, None)
    o = oracle.draft_lowrank(dn, u, x, k, dense_w=dense)
    assert np.array_equal(o["t"], oracle.linear(oracle.FMT_BF16, down, None, x,
                                                oracle.MODE_BF16))
    t2 = o["t"].copy()
    t2[0, 0] ^= 1                                     # a t one ulp away: its own logits
    c = oracle.draft_lowrank(dn, u, x, k, dense_w=dense, t=t2)
    assert np.array_equal(c["logits"].view(np.uint32),
                          oracle.gemv(oracle.FMT_BF16, up, None, t2).view(np.uint32))
    ex, dr = oracle.rescore(dense, x, o["ids"], o["vals"] > -np.inf)
    assert np.array_equal(o["exact"].view(np.uint32), ex.view(np.uint32))
    assert np.array_equal(o["draft"], dr)
