"""GPU parity on the full workloads, in the launch configuration the benchmark times:

  tiny_bf16       H=256,  V=4096,   1 row,  bf16 head, top-8 + argmax
  fp8_block_1row  H=5120, V=129280, 1 row,  FP8 E4M3 + E8M0 32x32 blocks, top-64 + argmax
  row_sweep       H=5120, V=129280, rows 1/5/10/15/16, the same head as bf16 and as FP8
                  blocks, top-64 + argmax
  two_stage       H=5120, V=129280, 16 rows, FP8 with a row scale + the dense bf16 head,
                  top cand_k=512 then the rescore
  edge            H=7168, V=163840, 16 rows, FP8 blocks, coarse-grid activations with many
                  exact ties, planted zero/NaN/+inf/-inf rows and a block of 32 identical
                  head rows, k in {1,22,31,32,33,512}

Checks at each: codes and scales of the GPU quantizer equal the oracle's; every logit
within tolerance of the oracle (the oracle computes all of them); the GPU top-k equals the
oracle's top-k of the GPU's own logits bit for bit; the ids follow the gap rule against the
oracle's logits; two-stage through the conditional oracle.  Every draft also runs on the
head's tiled copy (dh_tile_head, the layout the benchmark times), whose logits, ids, values
and drafts must equal the row-major head's bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from few_row_vocab_amd import dh
from gpu_util import dev, dev_u16, host, need_gpu, say
from parity import check_logits, check_topk, eligible
from test_gpu_core import check_topk_winner

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

_cache = {}


def workload(name):
    if name not in _cache:
        say(f"generating {name}")
        c = synth.CONFIGS[name]
        w = synth.head_bf16(name)
        x = synth.activations(name, max(c["rows"]))
        _cache.clear()
        _cache[name] = (c, w, x)
    return _cache[name]


def gpu_fp8(w, fmt):
    wd = dev_u16(w)
    codes, scale = dh.quantize(wd, fmt)
    del wd
    return codes, scale


def oracle_fp8(w, fmt):
    return oracle.quant_block32(w) if fmt == dh.FP8_BLOCK32 else oracle.quant_row(w)


def same_quant(codes, scale, oc, osc):
    gc = host(codes)
    assert np.array_equal(gc, oc), f"codes differ at {np.count_nonzero(gc != oc)} places"
    assert np.array_equal(host(scale).view(np.uint8), osc.view(np.uint8))


def exact_topk_on_gpu_logits(glog, ids, vals, k):
    oi, ov = oracle.topk(glog, k)
    assert np.array_equal(ids, oi)
    assert np.array_equal(vals.view(np.uint32), ov.view(np.uint32))


def same_outputs(a, b, names):
    for n in names:
        assert host(a[n]).tobytes() == host(b[n]).tobytes(), f"tiled head: {n} differs"


def run_one_stage(head, x, k, want, R, tiled=None):
    xd = dev_u16(x[:R])
    out = dh.draft(head, xd, k, keep_logits=True)
    if tiled is not None:
        same_outputs(out, dh.draft(tiled, xd, k, keep_logits=True),
                     ("logits", "ids", "vals", "draft"))
    torch.cuda.synchronize()
    glog, ids, vals, dr = (host(out[n]) for n in ("logits", "ids", "vals", "draft"))
    tols = check_logits(glog, want[:R])
    exact_topk_on_gpu_logits(glog, ids, vals, k)
    kinds = check_topk(ids, vals, want[:R], k, tols)
    assert np.array_equal(dr, ids[:, 0])
    check_topk(ids[:, :1], vals[:, :1], want[:R], 1, tols, what="argmax")
    return glog, kinds


def test_tiny_bf16():
    need_gpu()
    c, w, x = workload("tiny_bf16")
    want = oracle.gemv(oracle.FMT_BF16, w, None, x)
    head = dh.Head(dh.BF16, dev_u16(w))
    for k in c["ks"]:
        _, kinds = run_one_stage(head, x, k, want, 1)
        say(f"tiny_bf16 k={k}: {kinds}")


def test_fp8_block_1row():
    need_gpu()
    c, w, x = workload("fp8_block_1row")
    codes, scale = gpu_fp8(w, dh.FP8_BLOCK32)
    oc, osc = oracle_fp8(w, dh.FP8_BLOCK32)
    same_quant(codes, scale, oc, osc)
    want = oracle.gemv(oracle.FMT_FP8_BLOCK32, oc, osc, x)
    head = dh.Head(dh.FP8_BLOCK32, codes, scale)
    tiled = dh.tile(head)
    for k in c["ks"]:
        _, kinds = run_one_stage(head, x, k, want, 1, tiled)
        say(f"fp8_block_1row k={k}: {kinds}")


@pytest.mark.parametrize("fmt", ["bf16", "fp8_block32"])
def test_row_sweep(fmt):
    need_gpu()
    c, w, x = workload("row_sweep")
    if fmt == "bf16":
        head = dh.Head(dh.BF16, dev_u16(w))
        want = oracle.gemv(oracle.FMT_BF16, w, None, x)
    else:
        codes, scale = gpu_fp8(w, dh.FP8_BLOCK32)
        oc, osc = oracle_fp8(w, dh.FP8_BLOCK32)
        same_quant(codes, scale, oc, osc)
        head = dh.Head(dh.FP8_BLOCK32, codes, scale)
        want = oracle.gemv(oracle.FMT_FP8_BLOCK32, oc, osc, x)
    tiled = dh.tile(head)
    first = None
    for R in c["rows"]:
        glog, kinds = run_one_stage(head, x, 64, want, R, tiled)
        say(f"row_sweep {fmt} R={R}: {kinds}")
        if first is None:
            first = glog
        # batch invariance at full size: row 0 is bit-identical at every row count
        assert np.array_equal(glog[0].view(np.uint32), first[0].view(np.uint32))


def test_two_stage():
    need_gpu()
    c, w, x = workload("two_stage")
    k = c["ks"][0]
    codes, scale = gpu_fp8(w, dh.FP8_ROW)
    oc, osc = oracle_fp8(w, dh.FP8_ROW)
    same_quant(codes, scale, oc, osc)
    head = dh.Head(dh.FP8_ROW, codes, scale)
    dense = dh.Head(dh.BF16, dev_u16(w))
    xd = dev_u16(x)
    out = dh.draft(head, xd, k, dense=dense, keep_logits=True)
    same_outputs(out, dh.draft(dh.tile(head), xd, k, dense=dense, keep_logits=True),
                 ("logits", "ids", "vals", "exact", "draft"))
    torch.cuda.synchronize()
    glog, ids, vals, exact, dr = (host(out[n]) for n in ("logits", "ids", "vals", "exact", "draft"))
    want = oracle.gemv(oracle.FMT_FP8_ROW, oc, osc, x)
    tols = check_logits(glog, want)
    exact_topk_on_gpu_logits(glog, ids, vals, k)
    kinds = check_topk(ids, vals, want, k, tols)
    say(f"two_stage stage-1: {kinds}")
    oe, od = oracle.rescore(w, x, ids, vals > -np.inf)
    etol = check_logits(exact, oe, what="exact")
    for r in range(x.shape[0]):
        check_topk_winner(dr[r], oe[r], ids[r], etol[r], od[r])


def test_edge():
    need_gpu()
    c, w, x = workload("edge")
    codes, scale = gpu_fp8(w, dh.FP8_BLOCK32)
    oc, osc = oracle_fp8(w, dh.FP8_BLOCK32)
    same_quant(codes, scale, oc, osc)
    want = oracle.gemv(oracle.FMT_FP8_BLOCK32, oc, osc, x)
    head = dh.Head(dh.FP8_BLOCK32, codes, scale)
    tiled = dh.tile(head)
    hot = np.arange(synth.EDGE_HOT_BLOCK * 32, synth.EDGE_HOT_BLOCK * 32 + 32)
    for k in c["ks"]:
        glog, kinds = run_one_stage(head, x, k, want, 16, tiled)
        say(f"edge k={k}: {kinds}")
        assert np.all(np.isnan(glog[synth.EDGE_NAN_ROW]))
        assert np.all(glog[synth.EDGE_ZERO_ROW] == 0)
        # identical head rows give bit-identical logits in every row, so their exact ties
        # must resolve to the lower ids
        for r in range(16):
            hv = glog[r, hot]
            assert np.all(hv.view(np.uint32) == hv[0].view(np.uint32)) or np.all(np.isnan(hv))
    ids = host(dh.draft(head, dev_u16(x), 33)["ids"])
    assert np.array_equal(ids[synth.EDGE_HOT_ROW, :32], hot)
    assert np.all(ids[synth.EDGE_NAN_ROW] == 0)
    assert np.array_equal(ids[synth.EDGE_ZERO_ROW], np.arange(33))
