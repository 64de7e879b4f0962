"""Seeded random shapes across the whole range the library takes: rows 1..32, H a multiple
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

The oracle's work is bounded: V*H*R <= 1e9 multiply-adds and V*H <= 6e7 weights a case."""
import numpy as np
import pytest
import torch

import oracle
import synth
from few_row_vocab_amd import dh
from gpu_util import dev_u16, host, need_gpu, say
from parity import check_logits, check_topk
from test_gpu_core import FMTS, check_topk_winner, make_heads

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
