"""Seeded random shapes across the whole range the library takes.

dh_draft: rows 1..32, H a multiple
of 32 up to 32,768 (so the chunked GEMV for H > 8192 and the one-pass form for 17-32 rows
both come up), V up to 262,144 with ragged tails, k 1..512, the three head formats, row-major
and tiled heads, one- and two-stage drafts.  Each case checks

* the draft's logits against the oracle's GEMV (the logit rule of parity.py);
* the draft's ids, values and drafts against dh_topk on its own logits, bit for bit, and the
  logits against dh_gemv's, bit for bit;
* the ids against the oracle's top-k (the gap rule);
* one row of the call against the same row in a one-row call, bit for bit (the sums' order
  does not depend on the row count);
* in the two-stage form, the exact logits against the oracle's rescore of the GPU's own
  candidates and the draft against the oracle's winner (the conditional oracle).

dh_topk, dh_topk_mapped and dh_topk_softmax: rows 1..32, V up to 262,144, k 1..512, rows of
every planted kind (NaN, -inf, ties, zeros of both signs, subnormals, sorted runs, few
eligible entries), a strictly increasing id map half the time: bit for bit against the
oracle's top-k, the softmax statistics within their stated tolerance.

dh_linear: rows 1..32, K up to 32,768, N up to 40,000, the three formats and output modes.

dh_draft_mapped on a gathered subset head: rows 1..32, H up to 8,192, a subset of 1..V of
the head's ids, bf16 or FP8 row-scale, one- and two-stage, by the rules of test_gpu_subset.py.

dh_sample (the keyed pick) on dh_topk's lists: rows 1..32, V up to 262,144, k 1..512,
temperature 0..2, top-p and min-p drawn at random, by the rules of test_gpu_sample.py.

dh_rescore and dh_rescore_sync: thirty calls in a row through one sync buffer, rows 1..32,
H up to 32,768, 1..512 candidates a row with duplicates and ids outside the head planted:
the two bit-equal, the buffer all zero after each, the oracle's exact logits within tolerance.

dh_draft_lowrank: rows 1..32, H up to 8,192, rank 32..1,024, V up to 262,144, k 1..512, the
down and up heads in any of the three formats, one- and two-stage, by the rules of
test_gpu_lowrank.py.

The oracle's work is bounded: V*H*R <= 1e9 multiply-adds and V*H <= 6e7 weights a case."""
import numpy as np
import pytest
import torch

import oracle
import synth
from few_row_vocab_amd import dh
from gpu_util import dev, dev_u16, host, need_gpu, say
from test_gpu_rescore_sync import both
from parity import check_logits, check_topk
from test_gpu_core import FMTS, _planted, check_topk_winner, make_heads
from test_gpu_linear import _check_modes
from test_gpu_lowrank import run_and_check
from test_gpu_sample import check_picks
from test_gpu_subset import local_ids, oracle_subset
from test_gpu_softmax import check_softmax

pytestmark = pytest.mark.gpu

CASES = 120
MACS = 1e9
ELEMS = 6e7


def draw(seed):
    rng = np.random.default_rng(9100 + seed)
    fmt = ["bf16", "block", "row"][seed % 3]
    tiled = bool(rng.random() < 0.5)
    R = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 17, 24, 31, 32]))
    u = rng.random()
    if u < 0.7:
        H = 32 * int(rng.integers(1, 65))            # up to 2048
    elif u < 0.9:
        H = 32 * int(rng.integers(65, 257))          # up to 8192
    else:
        H = 32 * int(rng.integers(257, 1025))        # the chunked GEMV, up to 32768
    vmax = int(min(dh.MAX_VOCAB, MACS // (H * R), ELEMS // H))
    V = int(np.exp(rng.uniform(np.log(16), np.log(max(vmax, 17)))))
    V = max(1, min(V, vmax))
    k = int(rng.integers(1, min(dh.MAX_K, V) + 1))
    two = bool(rng.random() < 0.25)
    return fmt, tiled, R, H, V, k, two


@pytest.mark.parametrize("seed", range(CASES))
def test_random_shape_draft(seed):
    need_gpu()
    fmt, tiled, R, H, V, k, two = draw(seed)
    say(f"random shape {seed}: {fmt} tiled={tiled} R={R} H={H} V={V} k={k} two={two}")
    w = synth.random_head(V, H, seed=seed + 1, std=0.02)
    x = synth.random_acts(R, H, seed=seed + 2)
    gh, (ow, osc) = make_heads(fmt, w)
    if tiled and dh.tiled_bytes(gh.format, V, H):
        gh = dh.tile(gh)
    dense = dh.Head(dh.BF16, dev_u16(w)) if two else None
    xd = dev_u16(x)
    out = dh.draft(gh, xd, k, dense=dense, keep_logits=True)
    lg = dh.gemv(gh, xd)
    ids, vals, am = dh.topk(lg, k)
    r1 = R // 2
    one = dh.gemv(gh, xd[r1:r1 + 1].contiguous())
    torch.cuda.synchronize()
    logits = host(out["logits"])
    assert np.array_equal(logits.view(np.uint32), host(lg).view(np.uint32))
    assert np.array_equal(host(one)[0].view(np.uint32), logits[r1].view(np.uint32))
    gi, gv = host(out["ids"]), host(out["vals"])
    assert np.array_equal(gi, host(ids))
    assert np.array_equal(gv.view(np.uint32), host(vals).view(np.uint32))
    want = oracle.gemv(FMTS[fmt][1], ow, osc, x)
    tols = check_logits(logits, want)
    check_topk(gi, gv, want, k, tols)
    gd = host(out["draft"])
    if not two:
        assert np.array_equal(gd, host(am))
        return
    oe, od = oracle.rescore(w, x, gi, gv > -np.inf)
    etol = check_logits(host(out["exact"]), oe, what="exact")
    for r in range(R):
        check_topk_winner(gd[r], oe[r], gi[r], etol[r], od[r])


def _log_uniform(rng, lo, hi):
    return int(np.exp(rng.uniform(np.log(lo), np.log(hi + 1))))


@pytest.mark.parametrize("seed", range(60))
def test_random_shape_topk(seed):
    need_gpu()
    rng = np.random.default_rng(9300 + seed)
    R = int(rng.integers(1, dh.MAX_ROWS + 1))
    V = min(_log_uniform(rng, 1, dh.MAX_VOCAB), dh.MAX_VOCAB)
    k = int(rng.integers(1, min(dh.MAX_K, V) + 1))
    mapped = bool(rng.random() < 0.5)
    say(f"random top-k {seed}: R={R} V={V} k={k} mapped={mapped}")
    logits = _planted(R, V, seed=9400 + seed)
    d = dev(logits)
    if mapped:
        idmap = np.sort(rng.choice(2 * V + 7, V, replace=False)).astype(np.int32)
        ids, vals, am = dh.topk_mapped(d, k, dev(idmap))
        oi, ov = oracle.topk_mapped(logits, k, idmap)
    else:
        ids, vals, am = dh.topk(d, k)
        oi, ov = oracle.topk(logits, k)
        sm = dh.topk_softmax(d, k)
    gi, gv = host(ids), host(vals)
    assert np.array_equal(gi, oi)
    assert np.array_equal(gv.view(np.uint32), ov.view(np.uint32))
    assert np.array_equal(host(am), oi[:, 0])
    if not mapped:
        check_softmax(logits, k, sm)


@pytest.mark.parametrize("seed", range(40))
def test_random_shape_linear(seed):
    need_gpu()
    rng = np.random.default_rng(9500 + seed)
    fmt = ["bf16", "block", "row"][seed % 3]
    R = int(rng.integers(1, dh.MAX_ROWS + 1))
    K = 32 * _log_uniform(rng, 1, dh.MAX_HIDDEN // 32)
    K = min(K, dh.MAX_HIDDEN)
    N = max(1, min(_log_uniform(rng, 1, 40000), int(MACS // (K * R)), int(ELEMS // K)))
    say(f"random linear {seed}: {fmt} R={R} N={N} K={K}")
    w = synth.random_head(N, K, seed=9600 + seed, std=0.02)
    x = synth.random_acts(R, K, seed=9700 + seed)
    res = synth.random_acts(R, N, seed=9800 + seed, std=0.5)
    gh, (ow, osc) = make_heads(fmt, w)
    if rng.random() < 0.5 and dh.tiled_bytes(gh.format, N, K):
        gh = dh.tile(gh)
    _check_modes(gh, x, res, FMTS[fmt][1], ow, osc)


@pytest.mark.parametrize("seed", range(30))
def test_random_shape_lowrank(seed):
    need_gpu()
    rng = np.random.default_rng(9900 + seed)
    dfmt = ["bf16", "block", "row"][seed % 3]
    ufmt = ["bf16", "block", "row"][(seed // 3) % 3]
    R = int(rng.integers(1, dh.MAX_ROWS + 1))
    H = 32 * _log_uniform(rng, 1, 256)
    rk = 32 * _log_uniform(rng, 1, 32)
    V = max(1, min(_log_uniform(rng, 16, dh.MAX_VOCAB), dh.MAX_VOCAB, int(MACS // (rk * R)),
                   int(ELEMS // max(rk, H))))
    k = int(rng.integers(1, min(dh.MAX_K, V) + 1))
    two = bool(rng.random() < 0.3)
    label = f"random lowrank {seed}: {dfmt}/{ufmt} R={R} H={H} r={rk} V={V} k={k} two={two}"
    say(label)
    down = synth.random_head(rk, H, seed=10000 + seed, std=1 / np.sqrt(H))
    up = synth.random_head(V, rk, seed=10100 + seed, std=0.05)
    x = synth.random_acts(R, H, seed=10200 + seed)
    dense = synth.random_head(V, H, seed=10300 + seed, std=0.02) if two else None
    run_and_check(dfmt, ufmt, down, up, x, k, dense, label)


@pytest.mark.parametrize("seed", range(30))
def test_random_shape_mapped(seed):
    need_gpu()
    rng = np.random.default_rng(10400 + seed)
    fmt = ["bf16", "row"][seed % 2]
    R = int(rng.integers(1, dh.MAX_ROWS + 1))
    H = 32 * _log_uniform(rng, 1, 256)
    V = max(2, min(_log_uniform(rng, 16, dh.MAX_VOCAB), int(MACS // (H * R)), int(ELEMS // H)))
    n = int(rng.integers(1, V + 1))
    k = int(rng.integers(1, min(dh.MAX_K, n) + 1))
    two = bool(rng.random() < 0.3)
    say(f"random mapped {seed}: {fmt} R={R} H={H} V={V} n={n} k={k} two={two}")
    w = synth.random_head(V, H, seed=10500 + seed, std=0.02)
    x = synth.random_acts(R, H, seed=10600 + seed)
    gh, oh = make_heads(fmt, w)
    idmap = synth.token_ids(V, n, seed=10700 + seed)
    im = dev(idmap)
    sub = dh.gather_rows(gh, im)
    dense = dh.Head(dh.BF16, dev_u16(w)) if two else None
    xd = dev_u16(x)
    out = dh.draft_mapped(sub, im, xd, k, dense=dense, keep_logits=True)
    full = dh.gemv(gh, xd)
    torch.cuda.synchronize()
    glog, ids, vals, dr = (host(out[n_]) for n_ in ("logits", "ids", "vals", "draft"))
    assert np.array_equal(glog.view(np.uint32), host(full)[:, idmap].view(np.uint32))
    ofmt = FMTS[fmt][1]
    ow, osc = oracle_subset(ofmt, oh, idmap)
    want = oracle.gemv(ofmt, ow, osc, x)
    tols = check_logits(glog, want)
    oi, ov = oracle.topk_mapped(glog, k, idmap)
    assert np.array_equal(ids, oi)
    assert np.array_equal(vals.view(np.uint32), ov.view(np.uint32))
    check_topk(local_ids(ids, vals, idmap), vals, want, k, tols)
    if not two:
        assert np.array_equal(dr, ids[:, 0])
        return
    oe, od = oracle.rescore(w, x, ids, vals > -np.inf)
    etol = check_logits(host(out["exact"]), oe, what="exact")
    for r in range(R):
        check_topk_winner(dr[r], oe[r], ids[r], etol[r], od[r])


@pytest.mark.parametrize("seed", range(30))
def test_random_shape_sample(seed):
    need_gpu()
    rng = np.random.default_rng(10800 + seed)
    R = int(rng.integers(1, dh.MAX_ROWS + 1))
    V = min(_log_uniform(rng, 1, dh.MAX_VOCAB), dh.MAX_VOCAB)
    k = int(rng.integers(1, min(dh.MAX_K, V) + 1))
    T = 0.0 if rng.random() < 0.15 else float(rng.uniform(0.02, 2.0))
    top_p = 1.0 if rng.random() < 0.4 else float(rng.uniform(0.05, 1.0))
    min_p = 0.0 if rng.random() < 0.5 else float(rng.uniform(0.0, 0.5))
    key = int(rng.integers(0, 2**63)) * 2 + 1
    say(f"random sample {seed}: R={R} V={V} k={k} T={T:.3f} top_p={top_p:.3f} "
        f"min_p={min_p:.3f}")
    logits = _planted(R, V, seed=10900 + seed)
    ids, vals, _ = dh.topk(dev(logits), k)
    pos = rng.integers(0, 2**40, R).astype(np.int64)
    tok, kept = dh.sample(ids, vals, dev(pos), temperature=T, top_p=top_p, min_p=min_p,
                          seed=key)
    torch.cuda.synchronize()
    check_picks(host(ids), host(vals), T, top_p, min_p, key, pos, host(tok), host(kept))


def test_random_shape_rescore_sequence():
    need_gpu()
    rng = np.random.default_rng(11000)
    sync = dh.rescore_sync_buffer()
    for i in range(30):
        R = int(rng.integers(1, dh.MAX_ROWS + 1))
        H = 32 * _log_uniform(rng, 1, dh.MAX_HIDDEN // 32)
        H = min(H, dh.MAX_HIDDEN)
        V = max(1, min(_log_uniform(rng, 1, 1 << 20), int(ELEMS // H)))
        ck = int(rng.integers(1, dh.MAX_K + 1))
        say(f"random rescore {i}: R={R} H={H} V={V} ck={ck}")
        wd = synth.random_head(V, H, seed=11100 + i, std=0.02)
        x = synth.random_acts(R, H, seed=11200 + i)
        cand = rng.integers(0, V, (R, ck)).astype(np.int32)
        bad = rng.random((R, ck)) < 0.02                 # ids outside the head: NaN, never read
        cand[bad] = rng.choice([-1, V, V + 1000, np.iinfo(np.int32).max], int(bad.sum()))
        if ck > 1:
            cand[0, ck // 2:] = cand[0, 0]               # a run of one repeated id
        dense = dh.Head(dh.BF16, dev_u16(wd))
        e1, d1, e2, d2 = both(dense, dev_u16(x), dev(cand), sync)
        assert np.array_equal(e1.view(np.uint32), e2.view(np.uint32)), i
        assert np.array_equal(d1, d2), i
        assert not host(sync).any(), f"call {i} left its sync buffer non-zero"
        oe, od = oracle.rescore(wd, x, cand)
        tols = check_logits(e2, oe, what="exact")
        for r in range(R):
            check_topk_winner(d2[r], oe[r], cand[r], tols[r], od[r])
