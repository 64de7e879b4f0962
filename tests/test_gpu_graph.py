"""The projection captured in a HIP graph (torch.cuda.CUDAGraph on ROCm): every replay
equals the eager result bit for bit, with the program's own eager work and synchronizations
between replays.  The library allocates nothing and records no memset, so the whole draft
(one-stage, two-stage, subset, low-rank, with the keyed pick) can be captured."""
import numpy as np
import pytest
import torch

import synth
from few_row_vocab_amd import dh
from gpu_util import dev, dev_u16, host, need_gpu, say

pytestmark = pytest.mark.gpu


def _outs(R, k, V, dense):
    o = {"ids": torch.empty((R, k), dtype=torch.int32, device="cuda"),
         "vals": torch.empty((R, k), dtype=torch.float32, device="cuda"),
         "draft": torch.empty((R,), dtype=torch.int32, device="cuda"),
         "logits": torch.empty((R, V), dtype=torch.float32, device="cuda")}
    if dense:
        o["exact"] = torch.empty((R, k), dtype=torch.float32, device="cuda")
    return o


def _snap(o):
    return {n: host(t).copy() for n, t in o.items()}


def _same(a, b):
    for n in a:
        assert np.array_equal(a[n].view(np.uint8), b[n].view(np.uint8)), n


@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("two", [False, True])
def test_graph_replays_equal_eager(two, tiled):
    need_gpu()
    V, H, R, k = 20000, 1024, 16, 64
    w = synth.random_head(V, H, seed=5, std=0.02)
    wd = dev_u16(w)
    codes, scale = dh.quantize(wd, dh.FP8_BLOCK32 if not two else dh.FP8_ROW)
    head = dh.Head(dh.FP8_BLOCK32 if not two else dh.FP8_ROW, codes, scale)
    if tiled:
        head = dh.tile(head)
    dense = dh.Head(dh.BF16, wd) if two else None
    x = dev_u16(synth.random_acts(R, H, seed=6))
    ws = dh.workspace(R, V, k)
    pos = torch.arange(R, dtype=torch.int64, device="cuda")
    tok = torch.empty((R,), dtype=torch.int32, device="cuda")
    o = _outs(R, k, V, two)

    def step():
        dh.draft(head, x, k, dense=dense, ws=ws, out=o)
        dh.sample(o["ids"], o["vals"], pos, temperature=0.7, top_p=0.9, seed=3, token=tok,
                  with_kept=False)

    step()                                   # eager, also sets per-device kernel attributes
    torch.cuda.synchronize()
    want = _snap(o)
    want["token"] = host(tok).copy()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                               # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in o.values():
            t.fill_(0)
        tok.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snap(o)
        got["token"] = host(tok).copy()
        _same(want, got)
        # eager work between replays
        dh.gemv(head, x, o["logits"])
        torch.cuda.synchronize()
    say(f"graph two={two}: 4 replays equal eager")


def test_graph_subset_and_lowrank():
    need_gpu()
    V, H, R, k, n, rk = 12000, 512, 8, 32, 3000, 64
    w = synth.random_head(V, H, seed=7, std=0.02)
    wd = dev_u16(w)
    head = dh.Head(dh.FP8_ROW, *dh.quantize(wd, dh.FP8_ROW))
    im = dev(synth.token_ids(V, n, seed=8))
    sub = dh.gather_rows(head, im)
    down = dh.Head(dh.BF16, dev_u16(synth.random_head(rk, H, seed=9, std=H ** -0.5)))
    up = dh.Head(dh.BF16, dev_u16(synth.random_head(V, rk, seed=10, std=0.05)))
    x = dev_u16(synth.random_acts(R, H, seed=11))
    ws_s, ws_l = dh.workspace(R, n, k), dh.workspace(R, V, k)
    os_ = _outs(R, k, n, False)
    ol = _outs(R, k, V, False)
    ol["t"] = torch.empty((R, rk), dtype=torch.int16, device="cuda")

    def step():
        dh.draft_mapped(sub, im, x, k, ws=ws_s, out=os_)
        dh.draft_lowrank(down, up, x, k, ws=ws_l, out=ol)

    step()
    torch.cuda.synchronize()
    want = {**{"s_" + a: b for a, b in _snap(os_).items()},
            **{"l_" + a: b for a, b in _snap(ol).items()}}
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in list(os_.values()) + list(ol.values()):
            t.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {**{"s_" + a: b for a, b in _snap(os_).items()},
               **{"l_" + a: b for a, b in _snap(ol).items()}}
        _same(want, got)


@pytest.mark.parametrize("R,k", [(1, 64), (16, 512)])
def test_graph_topk_standalone(R, k):
    """dh_topk (the cut pass, then the merge), dh_topk_softmax (the same two kernels with the
    softmax statistics) and dh_rescore_sync (its sync buffer left zero by every call) in one
    graph: every replay equals the eager results."""
    need_gpu()
    V, H = 50000, 256
    rng = np.random.default_rng(R + k)
    lg = dev(rng.standard_normal((R, V)).astype(np.float32))
    wd = synth.random_head(V, H, seed=21, std=0.02)
    dense = dh.Head(dh.BF16, dev_u16(wd))
    x = dev_u16(synth.random_acts(R, H, seed=22))
    ws = dh.workspace(R, V, k)
    ws2 = dh.workspace(R, V, k)
    sync = dh.rescore_sync_buffer()
    o = {"ids": torch.empty((R, k), dtype=torch.int32, device="cuda"),
         "vals": torch.empty((R, k), dtype=torch.float32, device="cuda"),
         "am": torch.empty((R,), dtype=torch.int32, device="cuda"),
         "exact": torch.empty((R, k), dtype=torch.float32, device="cuda"),
         "draft": torch.empty((R,), dtype=torch.int32, device="cuda")}
    s = {}

    def step():
        dh.topk(lg, k, ws=ws, ids=o["ids"], vals=o["vals"], argmax=o["am"])
        i2, v2, a2, p2, l2 = dh.topk_softmax(lg, k, ws=ws2)
        s.update(i2=i2, v2=v2, p2=p2, l2=l2)
        dh.rescore(dense, x, o["ids"], exact=o["exact"], draft=o["draft"], sync=sync)

    step()
    torch.cuda.synchronize()
    want = _snap(o)
    want_s = _snap(s)
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        step()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in list(o.values()) + list(s.values()):
            t.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(want, _snap(o))
        _same(want_s, _snap(s))
        assert not host(sync).any(), rep
        dh.topk(lg, k, ws=ws)                # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("R", [1, 16])
def test_graph_linear_workspace(R):
    """dh_linear_ws on a linear wider than 8192 columns (its column chunks at once, then their
    sum in order) and dh_linear beside it, in every output mode, captured in one graph: every
    replay equals the eager results, and the two entries agree bit for bit."""
    need_gpu()
    N, K = 2051, 18432
    w = synth.random_head(N, K, seed=201, std=0.02)
    gr = dh.tile(dh.Head(dh.FP8_ROW, *dh.quantize(dev_u16(w).view(torch.bfloat16), dh.FP8_ROW)))
    x = dev_u16(synth.random_acts(R, K, seed=202))
    res = dev_u16(synth.random_acts(R, N, seed=203, std=0.5))
    ws = dh.linear_workspace(R, N, K)
    o = {"f32": torch.empty((R, N), dtype=torch.float32, device="cuda"),
         "bf16": torch.empty((R, N), dtype=torch.int16, device="cuda"),
         "add": torch.empty((R, N), dtype=torch.int16, device="cuda"),
         "plain": torch.empty((R, N), dtype=torch.float32, device="cuda")}

    def step():
        dh.linear(gr, x, dh.OUT_F32, out=o["f32"], ws=ws)
        dh.linear(gr, x, dh.OUT_BF16, out=o["bf16"], ws=ws)
        dh.linear(gr, x, dh.OUT_ADD_BF16, residual=res, out=o["add"], ws=ws)
        dh.linear(gr, x, dh.OUT_F32, out=o["plain"])

    step()
    torch.cuda.synchronize()
    want = _snap(o)
    assert np.array_equal(want["f32"].view(np.uint32), want["plain"].view(np.uint32))
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        step()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in o.values():
            t.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(want, _snap(o))
        dh.linear(gr, x, dh.OUT_F32, out=o["plain"], ws=ws)   # eager work between replays
        torch.cuda.synchronize()
