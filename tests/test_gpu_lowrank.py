"""GPU parity of dh_draft_lowrank (a low-rank stage 1, then the top-k and the rescore) against
the oracle's O15, through the C ABI.

 * t (the bf16 rank-r activations) is bit-identical to the GPU's own fp32 linear rounded on
   the host and within tol + 1 bf16 ulp of the oracle's t; the draft computes t split over
   workgroups (few tiles), dh_linear unsplit, so this also holds the split to the same bits;
 * the logits are within tolerance of the conditional oracle (O5 of `up` on the GPU's t);
   the top-k is bit-exact on the GPU's own logits and follows the gap rule on the
   conditional oracle's; the rescore follows the conditional oracle on the GPU's list;
 * dh_draft_lowrank equals dh_linear (bf16) -> dh_gemv -> dh_topk (-> dh_rescore) bit for bit;
 * the full-size workload: H=5120, V=129280, rank 512, 16 rows, cand_k=512, dense bf16 head.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from few_row_vocab_amd import dh
from gpu_util import dev_u16, host, need_gpu, say
from parity import check_logits, check_topk
from test_gpu_core import FMTS, check_topk_winner, make_heads
from test_gpu_linear import check_bf16, torch_bf16

pytestmark = pytest.mark.gpu


def run_and_check(dfmt, ufmt, down, up, x, k, dense_w, label):
    gd, (od, osd) = make_heads(dfmt, down)
    gu, (ou, osu) = make_heads(ufmt, up)
    xd = dev_u16(x)
    dense = dh.Head(dh.BF16, dev_u16(dense_w)) if dense_w is not None else None
    out = dh.draft_lowrank(gd, gu, xd, k, dense=dense, keep_logits=True)
    tf = dh.linear(gd, xd, dh.OUT_F32)
    torch.cuda.synchronize()
    t = host(out["t"]).view(np.uint16)
    glog, ids, vals, dr = (host(out[n]) for n in ("logits", "ids", "vals", "draft"))
    assert np.array_equal(t, torch_bf16(host(tf)))
    of_d, of_u = FMTS[dfmt][1], FMTS[ufmt][1]
    t_pre = oracle.linear(of_d, od, osd, x, oracle.MODE_F32)
    check_bf16(t, oracle.linear(of_d, od, osd, x, oracle.MODE_BF16), t_pre, f"{label} t")
    cond = oracle.draft_lowrank((of_d, od, osd), (of_u, ou, osu), x, k, t=t)
    tols = check_logits(glog, cond["logits"])
    oi, ov = oracle.topk(glog, k)
    assert np.array_equal(ids, oi)
    assert np.array_equal(vals.view(np.uint32), ov.view(np.uint32))
    kinds = check_topk(ids, vals, cond["logits"], k, tols)
    if dense_w is None:
        assert np.array_equal(dr, ids[:, 0])
    else:
        oe, od_ = oracle.rescore(dense_w, x, ids, vals > -np.inf)
        etol = check_logits(host(out["exact"]), oe, what="exact")
        for r in range(x.shape[0]):
            check_topk_winner(dr[r], oe[r], ids[r], etol[r], od_[r])
    say(f"{label}: {kinds}")
    return gd, gu, dense, out


@pytest.mark.parametrize("dfmt,ufmt", [("bf16", "bf16"), ("row", "row"), ("block", "bf16")])
@pytest.mark.parametrize("H,rk,V,R,k,two", [(256, 64, 5000, 1, 1, False),
                                            (1376, 96, 4133, 5, 64, True),
                                            (512, 512, 20000, 16, 512, True),
                                            (1088, 64, 3000, 32, 64, False)])
def test_lowrank_parity(dfmt, ufmt, H, rk, V, R, k, two):
    need_gpu()
    label = f"lowrank {dfmt}/{ufmt} H={H} r={rk} V={V} R={R} k={k} two={two}"
    say(label)
    down = synth.random_head(rk, H, seed=H + rk, std=1 / np.sqrt(H))
    up = synth.random_head(V, rk, seed=V + rk, std=0.05)
    x = synth.random_acts(R, H, seed=R + H)
    dense = synth.random_head(V, H, seed=V + H, std=0.02) if two else None
    run_and_check(dfmt, ufmt, down, up, x, k, dense, label)


def test_lowrank_equals_parts():
    need_gpu()
    H, rk, V, R, k = 1056, 128, 9000, 5, 64
    down = synth.random_head(rk, H, seed=21, std=1 / np.sqrt(H))
    up = synth.random_head(V, rk, seed=22, std=0.05)
    dense_w = synth.random_head(V, H, seed=23, std=0.02)
    x = synth.random_acts(R, H, seed=24)
    gd, gu = dh.Head(dh.BF16, dev_u16(down)), dh.Head(dh.BF16, dev_u16(up))
    dense = dh.Head(dh.BF16, dev_u16(dense_w))
    xd = dev_u16(x)
    o = dh.draft_lowrank(gd, gu, xd, k, dense=dense, keep_logits=True)
    t = dh.linear(gd, xd, dh.OUT_BF16)
    lg = dh.gemv(gu, t)
    i2, v2, _ = dh.topk(lg, k)
    e2, d2 = dh.rescore(dense, xd, i2)
    torch.cuda.synchronize()
    assert np.array_equal(host(o["t"]), host(t))
    assert np.array_equal(host(o["logits"]).view(np.uint32), host(lg).view(np.uint32))
    assert np.array_equal(host(o["ids"]), host(i2))
    assert np.array_equal(host(o["vals"]).view(np.uint32), host(v2).view(np.uint32))
    assert np.array_equal(host(o["exact"]).view(np.uint32), host(e2).view(np.uint32))
    assert np.array_equal(host(o["draft"]), host(d2))


def test_lowrank_refusals_on_device():
    need_gpu()
    H, rk, V, R, k = 256, 64, 1000, 2, 8
    gd = dh.Head(dh.BF16, dev_u16(synth.random_head(rk, H, seed=31)))
    gu = dh.Head(dh.BF16, dev_u16(synth.random_head(V, rk, seed=32)))
    bad_up = dh.Head(dh.BF16, dev_u16(synth.random_head(V, 96, seed=33)))
    xd = dev_u16(synth.random_acts(R, H, seed=34))
    with pytest.raises(dh.DHError):
        dh.draft_lowrank(gd, bad_up, xd, k)                       # up width != rank
    dense = dh.Head(dh.BF16, dev_u16(synth.random_head(V, rk, seed=35)))
    with pytest.raises(dh.DHError):
        dh.draft_lowrank(gd, gu, xd, k, dense=dense)              # dense width != H
    out = {"t": torch.zeros((R, rk + 8), dtype=torch.int16, device="cuda")[:, 1:rk + 1]}
    with pytest.raises((dh.DHError, ValueError)):
        dh.draft_lowrank(gd, gu, xd, k, out=out)                  # t not contiguous
    torch.cuda.synchronize()


@pytest.mark.slow
def test_lowrank_workload():
    need_gpu()
    name = "lowrank"
    c = synth.CONFIGS[name]
    say(f"generating {name}")
    down, up = synth.lowrank_factors(name)
    w = synth.head_bf16(name)
    x = synth.activations(name, max(c["rows"]))
    run_and_check("bf16", "bf16", down, up, x, c["ks"][0], w, "lowrank workload")
