"""dh_draft_noalloc (the draft on the library's fixed device scratch) against dh_draft on
the same inputs, through the C ABI: bit-equal outputs on two calls in a row on the same
stream, the second with a smaller input, so the second call runs on scratch the first one
left behind."""
import numpy as np
import pytest
import torch

import oracle
import synth
from few_row_vocab_amd import dh
from gpu_util import dev_u16, host, need_gpu, say
from parity import check_logits, check_topk

pytestmark = pytest.mark.gpu


def _outs(R, k, V, dense, logits):
    o = {"ids": torch.empty((R, k), dtype=torch.int32, device="cuda"),
         "vals": torch.empty((R, k), dtype=torch.float32, device="cuda"),
         "draft": torch.empty((R,), dtype=torch.int32, device="cuda")}
    if dense:
        o["exact"] = torch.empty((R, k), dtype=torch.float32, device="cuda")
    if logits:
        o["logits"] = torch.empty((R, V), dtype=torch.float32, device="cuda")
    return o


@pytest.mark.parametrize("two_stage", [False, True])
def test_noalloc_equals_draft_two_calls(two_stage):
    need_gpu()
    say(f"dh_draft_noalloc vs dh_draft, two_stage={two_stage}")
    cases = [(40000, 1024, 16, 64), (9000, 512, 3, 8)]        # the second call is smaller
    for i, (V, H, R, k) in enumerate(cases):
        w = synth.random_head(V, H, seed=31 + i, std=0.02)
        x = synth.random_acts(R, H, seed=41 + i)
        wd, xd = dev_u16(w), dev_u16(x)
        if two_stage:
            head = dh.Head(dh.FP8_ROW, *dh.quantize(wd, dh.FP8_ROW))
            dense = dh.Head(dh.BF16, wd)
        else:
            head = dh.tile(dh.Head(dh.FP8_BLOCK32, *dh.quantize(wd, dh.FP8_BLOCK32)))
            dense = None
        keep = i == 0                       # logits kept on the first call, in scratch on the second
        want = dh.draft(head, xd, k, dense=dense, keep_logits=keep)
        got = _outs(R, k, V, two_stage, keep)
        dh.draft_noalloc(head, xd, k, dense=dense, out=got)
        torch.cuda.synchronize()
        for name in want:
            assert torch.equal(got[name], want[name]), (i, name)
        if not two_stage and keep:
            oc, osc = oracle.quant_block32(w)
            ref = oracle.gemv(oracle.FMT_FP8_BLOCK32, oc, osc, x)
            tols = check_logits(host(got["logits"]), ref)
            check_topk(host(got["ids"]), host(got["vals"]), ref, k, tols)
        say(f"  call {i}: V={V} H={H} R={R} k={k} equal")


def test_noalloc_random_sequence():
    """Twelve calls in a row of seeded random shapes (rows 1..32, H up to 8192, V up to 2^18,
    k 1..512, three formats, row-major or tiled, one or two stages, logits kept or in the
    scratch), each on the scratch the previous one left behind: bit-equal to dh_draft."""
    need_gpu()
    rng = np.random.default_rng(4242)
    fmts = [dh.BF16, dh.FP8_BLOCK32, dh.FP8_ROW]
    for i in range(12):
        R = int(rng.integers(1, dh.MAX_ROWS + 1))
        H = 32 * int(np.exp(rng.uniform(0, np.log(256))))
        V = int(np.exp(rng.uniform(np.log(16), np.log(dh.MAX_VOCAB))))
        V = max(16, min(V, int(3e7 // H)))
        k = int(rng.integers(1, min(dh.MAX_K, V) + 1))
        two = bool(rng.random() < 0.3)
        keep = bool(rng.random() < 0.5)
        while dh.workspace_bytes(R, V, k) + 4096 > dh.NOALLOC_SCRATCH_BYTES:
            V //= 2                         # the top-k's workspace alone must fit the scratch
        k = min(k, V)
        if dh.workspace_bytes(R, V, k) + R * V * 4 + 4096 > dh.NOALLOC_SCRATCH_BYTES:
            keep = True                     # the logits would not fit beside the workspace
        f = fmts[i % 3]
        say(f"  noalloc sequence {i}: fmt={f} R={R} H={H} V={V} k={k} two={two} keep={keep}")
        w = synth.random_head(V, H, seed=500 + i, std=0.02)
        wd, xd = dev_u16(w), dev_u16(synth.random_acts(R, H, seed=600 + i))
        head = dh.Head(f, wd) if f == dh.BF16 else dh.Head(f, *dh.quantize(wd, f))
        if rng.random() < 0.5 and dh.tiled_bytes(head.format, V, H):
            head = dh.tile(head)
        dense = dh.Head(dh.BF16, wd) if two else None
        want = dh.draft(head, xd, k, dense=dense, keep_logits=keep)
        got = _outs(R, k, V, two, keep)
        dh.draft_noalloc(head, xd, k, dense=dense, out=got)
        torch.cuda.synchronize()
        for name in want:
            assert torch.equal(got[name], want[name]), (i, name)


def test_noalloc_refuses_beyond_its_scratch():
    need_gpu()
    V, H, R, k = 200000, 64, 32, 8
    w = torch.zeros((V, H), dtype=torch.int16, device="cuda")
    x = torch.zeros((R, H), dtype=torch.int16, device="cuda")
    with pytest.raises(dh.DHError) as e:
        dh.draft_noalloc(dh.Head(dh.BF16, w), x, k)
    assert e.value.status == 5
    # with the logits kept the same sizes fit
    o = dh.draft_noalloc(dh.Head(dh.BF16, w), x, k, keep_logits=True)
    torch.cuda.synchronize()
    assert torch.all(o["ids"] == torch.arange(k, dtype=torch.int32, device="cuda"))
