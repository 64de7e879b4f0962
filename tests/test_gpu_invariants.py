"""GPU self-consistency beyond the oracle: repeat determinism, batch invariance (a row's
logits do not depend on how many rows share the call -- the pages hold 1- and 16-row calls
byte-equal to the same rows inside a bigger call), concurrent streams equal serial, and
refused calls leaving device outputs untouched."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from few_row_vocab_amd import dh
from gpu_util import dev, dev_u16, host, need_gpu, say

pytestmark = pytest.mark.gpu


def _head(fmt, V, H, seed):
    w = synth.random_head(V, H, seed, std=0.02)
    wd = dev_u16(w)
    if fmt == dh.BF16:
        return dh.Head(dh.BF16, wd)
    c, s = dh.quantize(wd, fmt)
    return dh.Head(fmt, c, s)


@pytest.mark.parametrize("fmt", [dh.BF16, dh.FP8_BLOCK32, dh.FP8_ROW])
def test_batch_invariance_and_repeat(fmt):
    need_gpu()
    V, H = 6007, 5120
    head = _head(fmt, V, H, seed=51)
    x = dev_u16(synth.random_acts(16, H, seed=52))
    full = host(dh.gemv(head, x))
    again = host(dh.gemv(head, x))
    assert np.array_equal(full.view(np.uint32), again.view(np.uint32))
    for R in (1, 2, 5, 10, 15):
        for start in (0, 16 - R):
            part = host(dh.gemv(head, x[start:start + R].contiguous()))
            assert np.array_equal(part.view(np.uint32), full[start:start + R].view(np.uint32)), (R, start)


def test_draft_repeat_bit_equal():
    need_gpu()
    V, H, k = 20011, 2048, 512
    head = _head(dh.FP8_BLOCK32, V, H, seed=53)
    x = dev_u16(synth.random_acts(16, H, seed=54))
    a = dh.draft(head, x, k)
    b = dh.draft(head, x, k)
    torch.cuda.synchronize()
    for key in ("ids", "draft"):
        assert torch.equal(a[key], b[key])
    assert torch.equal(a["vals"].view(torch.int32), b["vals"].view(torch.int32))


def test_two_streams_equal_serial():
    need_gpu()
    V, H, k = 30000, 4096, 64
    h1 = _head(dh.FP8_BLOCK32, V, H, seed=55)
    h2 = _head(dh.BF16, V, H, seed=56)
    x = dev_u16(synth.random_acts(16, H, seed=57))
    s1 = dh.draft(h1, x, k)
    s2 = dh.draft(h2, x, k)
    torch.cuda.synchronize()
    st1, st2 = torch.cuda.Stream(), torch.cuda.Stream()
    ws1, ws2 = dh.workspace(16, V, k), dh.workspace(16, V, k)
    torch.cuda.synchronize()
    with torch.cuda.stream(st1):
        c1 = dh.draft(h1, x, k, ws=ws1)
    with torch.cuda.stream(st2):
        c2 = dh.draft(h2, x, k, ws=ws2)
    torch.cuda.synchronize()
    for a, b in ((s1, c1), (s2, c2)):
        assert torch.equal(a["ids"], b["ids"]) and torch.equal(a["draft"], b["draft"])
        assert torch.equal(a["vals"].view(torch.int32), b["vals"].view(torch.int32))


def test_refusals_on_device_buffers_leave_outputs_untouched():
    need_gpu()
    V, H, k, R = 1000, 64, 8, 2
    head = _head(dh.FP8_BLOCK32, V, H, seed=58)
    x = dev_u16(synth.random_acts(R, H, seed=59))
    L = dh.lib()
    out = torch.full((R, V), 7.0, device="cuda")
    h = head._c()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.dh_gemv(ctypes.byref(h), ctypes.c_void_p(x.data_ptr()), 33, ctypes.c_void_p(out.data_ptr()), st) == 2
    ids = torch.full((R, k), 5, dtype=torch.int32, device="cuda")
    vals = torch.full((R, k), 5.0, device="cuda")
    ws = dh.workspace(R, V, k)
    assert L.dh_topk(ctypes.c_void_p(out.data_ptr()), R, V, 513, ctypes.c_void_p(ids.data_ptr()),
                     ctypes.c_void_p(vals.data_ptr()), None, ctypes.c_void_p(ws.data_ptr()),
                     ws.numel(), st) == 2
    assert L.dh_topk(ctypes.c_void_p(out.data_ptr()), R, V, k, ctypes.c_void_p(ids.data_ptr()),
                     ctypes.c_void_p(vals.data_ptr()), None, ctypes.c_void_p(ws.data_ptr()),
                     16, st) == 3
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(ids == 5) and torch.all(vals == 5.0)
    with pytest.raises(dh.DHError):
        dh.topk(out, 0)
