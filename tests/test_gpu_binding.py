"""The Python binding refuses tensors whose shape or dtype does not match what the library
would read or write through their pointers (the C ABI takes bare pointers and cannot check
sizes), before anything is launched."""
import numpy as np
import pytest
import torch

import synth
from few_row_vocab_amd import dh
from gpu_util import dev_u16, need_gpu

pytestmark = pytest.mark.gpu


def test_binding_shape_checks():
    need_gpu()
    V, H, R, k = 300, 64, 3, 8
    w = dev_u16(synth.random_head(V, H, seed=1))
    head = dh.Head(dh.BF16, w)
    x = dev_u16(synth.random_acts(R, H, seed=2))
    small = torch.zeros((R, V - 1), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        dh.gemv(head, x, small)                                   # logits one column short
    with pytest.raises(ValueError):
        dh.gemv(head, x[:, :32].contiguous())                     # x narrower than H
    with pytest.raises(TypeError):
        dh.linear(head, x, dh.OUT_BF16, out=torch.zeros((R, V), device="cuda"))   # f32 out
    with pytest.raises(ValueError):
        dh.linear(head, x, dh.OUT_ADD_BF16,
                  residual=torch.zeros((R, V + 1), dtype=torch.int16, device="cuda"))
    lg = dh.gemv(head, x)
    with pytest.raises(ValueError):
        dh.topk(lg, k, ids=torch.zeros((R, k - 1), dtype=torch.int32, device="cuda"))
    with pytest.raises(TypeError):
        dh.topk(lg, k, ws=torch.zeros(dh.workspace_bytes(R, V, k) // 4, dtype=torch.int32,
                                      device="cuda"))
    ids, vals, _ = dh.topk(lg, k)
    with pytest.raises(ValueError):
        dh.sample(ids, vals, torch.zeros(R + 1, dtype=torch.int64, device="cuda"))
    with pytest.raises(ValueError):
        dh.draft(head, x, k, out={"ids": torch.zeros((R, k + 1), dtype=torch.int32,
                                                     device="cuda")})
    codes, scale = dh.quantize(w, dh.FP8_ROW)
    with pytest.raises(ValueError):
        dh.gemv(dh.Head(dh.FP8_ROW, codes, scale[:-1]), x)        # row scales one short
    torch.cuda.synchronize()


def test_draft_on_a_side_stream_with_a_temporary_workspace(monkeypatch):
    """dh.draft(stream=s) with ws=None allocates its temporary workspace (which holds the
    logits when they are not kept) on s, so memory the current stream allocates right after
    the call cannot be that workspace while s still runs the draft."""
    need_gpu()
    V, H, R, k = 60000, 1024, 4, 64
    head = dh.Head(dh.BF16, dev_u16(synth.random_head(V, H, seed=11, std=0.02)))
    x = dev_u16(synth.random_acts(R, H, seed=12))
    want = dh.draft(head, x, k)
    torch.cuda.synchronize()
    made = []
    orig = dh.workspace

    def spy(*a, **kw):
        ws = orig(*a, **kw)
        made.append((ws.data_ptr(), ws.numel()))
        return ws

    monkeypatch.setattr(dh, "workspace", spy)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        a = torch.ones((2048, 2048), device="cuda")
        for _ in range(6):                                     # keeps the side stream busy
            a = (a @ a) / 2048.0
    got = dh.draft(head, x, k, stream=side)
    assert len(made) == 1
    # the current stream now allocates and writes as much memory as the workspace held
    junk = [torch.full((made[0][1],), 0xFF, dtype=torch.uint8, device="cuda")
            for _ in range(3)]
    for j in junk:
        lo, hi = j.data_ptr(), j.data_ptr() + j.numel()
        assert hi <= made[0][0] or lo >= made[0][0] + made[0][1]
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for name in ("ids", "vals", "draft"):
        assert torch.equal(got[name], want[name]), name
