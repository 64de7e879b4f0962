"""GPU parity of the draft-vocabulary subset head (dh_gather_rows, dh_topk_mapped,
dh_draft_mapped) against the oracle's O12/O13, through the C ABI.

 * gather: the subset head's codes, bf16 bits and row scales equal the oracle's bit for bit,
   duplicates and out-of-range ids included, for ragged counts and widths up to the maximum;
 * mapped top-k: bit-exact against the oracle's mapped top-k on planted logits (ties, NaN,
   -inf, fewer eligible entries than k) over several chunks and a ragged tail;
 * mapped draft: the subset's GPU logits equal the full head's GPU logits at the subset's ids
   bit for bit (a row's sums do not depend on the head it sits in), they are within the
   logit tolerance of the oracle, the top-k is bit-exact on the GPU's own logits and follows
   the gap rule on the oracle's, and in the two-stage form the full-vocabulary rescore
   follows the conditional oracle;
 * the full-size subset workload: 49,152 of 131,072 ids of an FP8 head of width 4,096, 1 and
   16 rows, k in {1, 64, 512}.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from few_row_vocab_amd import dh
from gpu_util import dev, dev_u16, host, need_gpu, say
from parity import check_logits, check_topk
from test_gpu_core import _planted, check_topk_winner, make_heads

pytestmark = pytest.mark.gpu


def local_ids(ids, vals, idmap):
    """Token ids -> subset columns (pads stay 0), for the gap rule on subset logits."""
    j = np.searchsorted(idmap, ids)
    return np.where(vals > -np.inf, j, 0).astype(np.int32)


def oracle_subset(fmt, oh, ids):
    ow, osc = oh
    return oracle.subset_rows(fmt, ow, osc, ids)


@pytest.mark.parametrize("fmt", ["bf16", "row"])
@pytest.mark.parametrize("V,H,n", [(70, 32, 1), (1000, 96, 3), (4133, 1376, 1001),
                                   (515, 8192, 77), (2051, 4096, 2050)])
def test_gather_rows_bit_exact(fmt, V, H, n):
    need_gpu()
    say(f"gather {fmt} V={V} H={H} n={n}")
    w = synth.random_head(V, H, seed=V + H, std=0.02)
    gh, oh = make_heads(fmt, w)
    rng = np.random.default_rng(n)
    ids = rng.integers(0, V, n).astype(np.int32)                 # duplicates allowed
    if n > 2:
        ids[[0, n // 2, n - 1]] = [-1, V, np.iinfo(np.int32).max]  # out of range: zero rows
    sub = dh.gather_rows(gh, dev(ids))
    torch.cuda.synchronize()
    ofmt = oracle.FMT_BF16 if fmt == "bf16" else oracle.FMT_FP8_ROW
    ow, osc = oracle_subset(ofmt, oh, ids)
    gw = host(sub.weight)
    if fmt == "bf16":
        gw = gw.view(np.uint16)
    assert np.array_equal(gw, ow)
    if fmt == "row":
        assert np.array_equal(host(sub.scale).view(np.uint32), osc.view(np.uint32))
    else:
        assert sub.scale is None


def test_gather_rows_refusals_on_device():
    need_gpu()
    V, H = 256, 64
    w = synth.random_head(V, H, seed=3, std=0.02)
    gh, _ = make_heads("block", w)
    ids = dev(np.arange(8, dtype=np.int32))
    with pytest.raises(dh.DHError) as e:
        dh.gather_rows(gh, ids)
    assert e.value.status == 2
    rh, _ = make_heads("row", w)
    out = torch.zeros((8, H), dtype=torch.uint8, device="cuda")
    h = rh._c()
    # the scale output is required for per-row FP8
    st = dh.lib().dh_gather_rows(ctypes.byref(h), dh._ptr(ids), 8, dh._ptr(out), None,
                                 dh._stream(None))
    assert st == 1
    torch.cuda.synchronize()
    assert not host(out).any()


@pytest.mark.parametrize("V", [70, 4097, 20000])
@pytest.mark.parametrize("k", [1, 8, 9, 64, 512])
def test_topk_mapped_bit_exact(V, k):
    need_gpu()
    if k > V:
        pytest.skip("k > V is refused")
    say(f"topk_mapped V={V} k={k}")
    logits = _planted(16, V, seed=V * 7 + k)
    idmap = synth.token_ids(262144, V, seed=V + k)
    ids, vals, am = dh.topk_mapped(dev(logits), k, dev(idmap))
    oi, ov = oracle.topk_mapped(logits, k, idmap)
    gi, gv = host(ids), host(vals)
    assert np.array_equal(gi, oi)
    assert np.array_equal(gv.view(np.uint32), ov.view(np.uint32))
    assert np.array_equal(host(am), oi[:, 0])
    # the unmapped top-k through the same map gives the same lists
    li, lv, _ = (host(t) if t is not None else None for t in dh.topk(dev(logits), k))
    real = lv > -np.inf
    assert np.array_equal(gi[real], idmap[li[real]]) and np.all(gi[~real] == 0)


@pytest.mark.parametrize("fmt,two", [("bf16", False), ("row", False), ("row", True),
                                     ("bf16", True)])
@pytest.mark.parametrize("R,k", [(1, 1), (5, 64), (16, 512)])
def test_draft_mapped_parity(fmt, two, R, k):
    need_gpu()
    V, H, n = 5000, 256, 1531
    say(f"draft_mapped {fmt} two={two} R={R} k={k}")
    w = synth.random_head(V, H, seed=81, std=0.02)
    x = synth.random_acts(R, H, seed=82)
    gh, oh = make_heads(fmt, w)
    idmap = synth.token_ids(V, n, seed=83)
    im = dev(idmap)
    sub = dh.gather_rows(gh, im)
    dense = dh.Head(dh.BF16, dev_u16(w)) if two else None
    xd = dev_u16(x)
    out = dh.draft_mapped(sub, im, xd, k, dense=dense, keep_logits=True)
    full = dh.gemv(gh, xd)
    torch.cuda.synchronize()
    glog, ids, vals, dr = (host(out[n_]) for n_ in ("logits", "ids", "vals", "draft"))
    # the subset's logits are the full head's at the subset's ids, bit for bit
    assert np.array_equal(glog.view(np.uint32), host(full)[:, idmap].view(np.uint32))
    ofmt = oracle.FMT_BF16 if fmt == "bf16" else oracle.FMT_FP8_ROW
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


def test_draft_mapped_equals_parts():
    """dh_draft_mapped == dh_topk_mapped(dh_gemv(subset)) bit for bit."""
    need_gpu()
    V, H, n, R, k = 9000, 1056, 4099, 5, 64
    w = synth.random_head(V, H, seed=91, std=0.02)
    x = synth.random_acts(R, H, seed=92)
    gh, _ = make_heads("row", w)
    im = dev(synth.token_ids(V, n, seed=93))
    sub = dh.gather_rows(gh, im)
    xd = dev_u16(x)
    o = dh.draft_mapped(sub, im, xd, k, keep_logits=True)
    lg = dh.gemv(sub, xd)
    i2, v2, a2 = dh.topk_mapped(lg, k, im)
    torch.cuda.synchronize()
    assert np.array_equal(host(o["logits"]).view(np.uint32), host(lg).view(np.uint32))
    assert np.array_equal(host(o["ids"]), host(i2))
    assert np.array_equal(host(o["vals"]).view(np.uint32), host(v2).view(np.uint32))
    assert np.array_equal(host(o["draft"]), host(a2))


@pytest.mark.slow
def test_subset_head_workload():
    """The full-size subset workload, in the launch configuration the benchmark times."""
    need_gpu()
    name = "subset_head"
    c = synth.CONFIGS[name]
    V, H, n = c["V"], c["H"], c["n_draft"]
    say(f"generating {name}")
    w = synth.head_bf16(name)
    x = synth.activations(name, max(c["rows"]))
    idmap = synth.draft_ids(name)
    wd = dev_u16(w)
    codes, scale = dh.quantize(wd, dh.FP8_ROW)
    del wd
    oc, osc = oracle.quant_row(w)
    assert np.array_equal(host(codes), oc)
    assert np.array_equal(host(scale).view(np.uint32), osc.view(np.uint32))
    full = dh.Head(dh.FP8_ROW, codes, scale)
    im = dev(idmap)
    sub = dh.gather_rows(full, im)
    ow, osub = oracle.subset_rows(oracle.FMT_FP8_ROW, oc, osc, idmap)
    assert np.array_equal(host(sub.weight), ow)
    assert np.array_equal(host(sub.scale).view(np.uint32), osub.view(np.uint32))
    want = oracle.gemv(oracle.FMT_FP8_ROW, ow, osub, x)
    for R in c["rows"]:
        xd = dev_u16(x[:R])
        full_l = host(dh.gemv(full, xd))
        for k in c["ks"]:
            out = dh.draft_mapped(sub, im, xd, k, keep_logits=True)
            torch.cuda.synchronize()
            glog, ids, vals, dr = (host(out[q]) for q in ("logits", "ids", "vals", "draft"))
            assert np.array_equal(glog.view(np.uint32), full_l[:, idmap].view(np.uint32))
            tols = check_logits(glog, want[:R])
            oi, ov = oracle.topk_mapped(glog, k, idmap)
            assert np.array_equal(ids, oi)
            assert np.array_equal(vals.view(np.uint32), ov.view(np.uint32))
            kinds = check_topk(local_ids(ids, vals, idmap), vals, want[:R], k, tols)
            assert np.array_equal(dr, ids[:, 0])
            say(f"subset_head R={R} k={k}: {kinds}")
