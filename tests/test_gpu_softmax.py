"""GPU parity of dh_topk_softmax (the top-k with each row's softmax statistics) against the
oracle's O16, through the C ABI.

 * ids and values bit-exact with the oracle's top-k (and with dh_topk);
 * probabilities within a relative 2e-5 of the oracle's, plus one subnormal quantum (2^-149)
   for probabilities below 2^-126 (pads exactly 0), lse within
   2e-5 * max(1, |lse|), infinities equal.  The bound: z is an fp32 sum of at most 2^18
   positive terms along a path of at most ~40 additions (16 a thread, 6 butterfly levels, 4
   waves of a chunk, 4 chunks a lane, 6 levels), about 3e-6 relative, plus expf's 1 ulp and
   the rounding of l - m, which is |l - m| * 2^-24 relative (6e-6 at |l - m| = 100);
 * planted rows of every kind (NaN, +-inf, ties, subnormals, rows without an eligible
   logit) and the FP8 head's own logits at 16 rows.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from few_row_vocab_amd import dh
from gpu_util import dev, dev_u16, host, need_gpu, say
from test_gpu_core import _planted, make_heads

pytestmark = pytest.mark.gpu
RTOL = 2e-5


def check_softmax(logits, k, got):
    ids, vals, am, probs, lse = (host(t) for t in got)
    oi, ov, op, ol = oracle.topk_softmax(logits, k)
    assert np.array_equal(ids, oi)
    assert np.array_equal(vals.view(np.uint32), ov.view(np.uint32))
    assert np.array_equal(am, oi[:, 0])
    inf = np.isinf(ol)
    assert np.array_equal(lse[inf], ol[inf])
    fin = ~inf
    err = np.abs(lse[fin].astype(np.float64) - ol[fin])
    assert np.all(err <= RTOL * np.maximum(1.0, np.abs(ol[fin]))), float(err.max())
    pad = vals == -np.inf
    assert np.all(probs[pad] == 0) and np.all(op[pad] == 0)
    # a probability below 2^-126 is subnormal: each side rounds it to a multiple of 2^-149
    err = np.abs(probs[~pad].astype(np.float64) - op[~pad])
    assert np.all(err <= RTOL * op[~pad] + 2.0**-149), float((err - RTOL * op[~pad]).max())


@pytest.mark.parametrize("V", [70, 4097, 20000, 163840])
@pytest.mark.parametrize("k", [1, 8, 64, 512])
def test_topk_softmax_planted(V, k):
    need_gpu()
    if k > V:
        pytest.skip("k > V is refused")
    say(f"topk_softmax V={V} k={k}")
    logits = _planted(16, V, seed=V * 3 + k)
    d = dev(logits)
    got = dh.topk_softmax(d, k)
    i2, v2, _ = dh.topk(d, k)
    torch.cuda.synchronize()
    assert torch.equal(got[0], i2) and torch.equal(got[1].view(torch.int32), v2.view(torch.int32))
    check_softmax(logits, k, got)


def test_topk_softmax_head_logits():
    need_gpu()
    V, H, R, k = 129280, 5120, 16, 64
    w = synth.head_bf16("row_sweep")
    x = synth.activations("row_sweep", R)
    gh, _ = make_heads("block", w)
    lg = dh.gemv(gh, dev_u16(x))
    got = dh.topk_softmax(lg, k)
    torch.cuda.synchronize()
    glog = host(lg)
    check_softmax(glog, k, got)
    conf = host(got[3])[:, 0]
    say(f"top-1 confidence of the 16 rows: {np.round(conf, 4).tolist()}")


def test_topk_softmax_refusals():
    need_gpu()
    R, V, k = 2, 1000, 8
    d = dev(np.zeros((R, V), np.float32))
    ws = dh.workspace(R, V, k)
    ids = torch.zeros((R, k), dtype=torch.int32, device="cuda")
    vals = torch.zeros((R, k), device="cuda")
    probs = torch.full((R, k), 7.0, device="cuda")
    L = dh.lib()
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = dh._stream(None)
    assert L.dh_topk_softmax(p(d), R, V, k, p(ids), p(vals), None, p(probs), None, p(ws),
                             ws.numel(), st) == 1            # lse missing
    assert L.dh_topk_softmax(p(d), R, V, k, p(ids), p(vals), None, p(probs), p(ids), p(ws),
                             ws.numel(), st) == 1            # lse overlaps ids
    torch.cuda.synchronize()
    assert bool((probs == 7.0).all())


def test_topk_softmax_preallocated_outputs():
    """The binding's `out` dict: the same bits as freshly allocated outputs, written in place
    (what a graph-captured caller passes), two calls in a row on different k."""
    need_gpu()
    R, V = 16, 20000
    logits = _planted(R, V, seed=77)
    d = dev(logits)
    for k in (64, 512):
        ws = dh.workspace(R, V, k)
        o = {"ids": torch.empty((R, k), dtype=torch.int32, device="cuda"),
             "vals": torch.empty((R, k), dtype=torch.float32, device="cuda"),
             "probs": torch.empty((R, k), dtype=torch.float32, device="cuda"),
             "lse": torch.empty((R,), dtype=torch.float32, device="cuda"),
             "argmax": torch.empty((R,), dtype=torch.int32, device="cuda")}
        got = dh.topk_softmax(d, k, ws=ws, out=o)
        ref = dh.topk_softmax(d, k)
        torch.cuda.synchronize()
        assert got[0] is o["ids"] and got[3] is o["probs"] and got[4] is o["lse"]
        for a, b in zip(got, ref):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32))
        check_softmax(logits, k, got)


@pytest.mark.parametrize("R", [1, 16, 32])
def test_topk_softmax_largest_vocabulary(R):
    """The largest vocabulary the top-k takes (V = 262,144) at k = 512: at one row the cut
    pass's 256 chunks a row, from 16 rows on its largest chunks (64 a row, 4096 logits)."""
    need_gpu()
    V, k = 262144, 512
    say(f"topk_softmax V={V} R={R}")
    logits = _planted(R, V, seed=R + 262)
    d = dev(logits)
    got = dh.topk_softmax(d, k)
    i2, v2, _ = dh.topk(d, k)
    torch.cuda.synchronize()
    assert torch.equal(got[0], i2) and torch.equal(got[1].view(torch.int32), v2.view(torch.int32))
    check_softmax(logits, k, got)
