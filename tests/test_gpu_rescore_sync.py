"""dh_rescore_sync, the one-launch rescore: the same exact logits and drafts as dh_rescore bit
for bit, the oracle's logits within tolerance, and a sync buffer that every call leaves all
zero -- across calls of different sizes in a row and across HIP graph replays."""
import numpy as np
import pytest
import torch

import oracle
import synth
from few_row_vocab_amd import dh
from gpu_util import dev, dev_u16, host, need_gpu, say
from parity import check_logits
from test_gpu_core import check_topk_winner

pytestmark = pytest.mark.gpu


def special_case(V, H, R, ck, seed):
    """Head, activations and candidates with the rescore's special cases planted: an exact
    tie between identical rows, ids outside the head, a row of one repeated id, a NaN row."""
    wd = synth.random_head(V, H, seed=seed, std=0.02)
    wd[100] = wd[200]
    x = synth.random_acts(R, H, seed=seed + 1)
    rng = np.random.default_rng(seed + 2)
    cand = rng.integers(0, V, (R, ck)).astype(np.int32)
    if ck >= 2:
        cand[0, :2] = [200, 100]
    if R >= 2 and ck >= 5:
        cand[1, 3] = V + 7
        cand[1, 4] = -2
    if R >= 3:
        cand[2, :] = cand[2, 0]
    if R >= 4:
        x[3, 5] = 0x7FC0
    return wd, x, cand


def both(dense, xd, cd, sync):
    e1, d1 = dh.rescore(dense, xd, cd)
    e2, d2 = dh.rescore(dense, xd, cd, sync=sync)
    torch.cuda.synchronize()
    return host(e1), host(d1), host(e2), host(d2)


@pytest.mark.parametrize("V,H,R,ck", [(3000, 544, 4, 37), (2000, 1024, 32, 512), (700, 256, 1, 1),
                                      (1500, 16384, 5, 21)])
def test_rescore_sync_equals_rescore_and_oracle(V, H, R, ck):
    need_gpu()
    say(f"rescore_sync V={V} H={H} R={R} ck={ck}")
    wd, x, cand = special_case(V, H, R, ck, seed=V + ck)
    dense = dh.Head(dh.BF16, dev_u16(wd))
    sync = dh.rescore_sync_buffer()
    e1, d1, e2, d2 = both(dense, dev_u16(x), dev(cand), sync)
    assert np.array_equal(e1.view(np.uint32), e2.view(np.uint32))
    assert np.array_equal(d1, d2)
    assert not host(sync).any(), "the call left its sync buffer non-zero"
    oe, od = oracle.rescore(wd, x, cand)
    tols = check_logits(e2, oe, what="exact")
    for r in range(R):
        check_topk_winner(d2[r], oe[r], cand[r], tols[r], od[r])


def test_rescore_sync_calls_in_a_row():
    """One sync buffer through calls of 32, 5, 16 and 1 rows: each equals dh_rescore."""
    need_gpu()
    V, H = 5000, 1024
    wd = synth.random_head(V, H, seed=71, std=0.02)
    dense = dh.Head(dh.BF16, dev_u16(wd))
    sync = dh.rescore_sync_buffer()
    rng = np.random.default_rng(72)
    for R, ck in ((32, 512), (5, 64), (16, 300), (1, 7)):
        x = synth.random_acts(R, H, seed=73 + R)
        cand = rng.integers(0, V, (R, ck)).astype(np.int32)
        e1, d1, e2, d2 = both(dense, dev_u16(x), dev(cand), sync)
        assert np.array_equal(e1.view(np.uint32), e2.view(np.uint32)), (R, ck)
        assert np.array_equal(d1, d2), (R, ck)
        assert not host(sync).any(), (R, ck)


def test_rescore_sync_graph_replays():
    """Three captured calls over different candidate sets, replayed three times with eager
    work between replays: every replay equals the eager results."""
    need_gpu()
    V, H, R, ck = 4000, 512, 16, 128
    wd = synth.random_head(V, H, seed=81, std=0.02)
    dense = dh.Head(dh.BF16, dev_u16(wd))
    xd = dev_u16(synth.random_acts(R, H, seed=82))
    rng = np.random.default_rng(83)
    cands = [dev(rng.integers(0, V, (R, ck)).astype(np.int32)) for _ in range(3)]
    want = [dh.rescore(dense, xd, c) for c in cands]
    torch.cuda.synchronize()
    want = [(host(e), host(d)) for e, d in want]
    sync = dh.rescore_sync_buffer()
    outs = [(torch.empty((R, ck), dtype=torch.float32, device="cuda"),
             torch.empty((R,), dtype=torch.int32, device="cuda")) for _ in range(3)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for c, (e, d) in zip(cands, outs):
                dh.rescore(dense, xd, c, exact=e, draft=d, sync=sync)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        for e, d in outs:
            e.fill_(-1.0)
            d.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (we, wdr), (e, d) in zip(want, outs):
            assert np.array_equal(host(e).view(np.uint32), we.view(np.uint32)), rep
            assert np.array_equal(host(d), wdr), rep
        assert not host(sync).any(), rep
        dh.rescore(dense, xd, cands[rep], sync=sync)   # eager work between replays
        torch.cuda.synchronize()
