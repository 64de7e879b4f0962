"""GPU parity of 17..32-row calls (two 16-row MFMA column blocks per weight tile) through the
C ABI, for the three weight formats.

 * logits within tolerance of the oracle, over tiles, ragged tails and H up to 4096 (one pass);
 * the pages' bit-equality across row counts: each row of a 17..32-row call equals the same
   row of a 1-row and of a 16-row call bit for bit;
 * dh_linear's output modes, dh_draft (top-k of 32 rows) and the subset head at 32 rows;
 * H = 5120 (one pass for FP8 heads) and above (two 16-row launches): the same parity and
   bit equality.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from few_row_vocab_amd import dh
from gpu_util import dev, dev_u16, host, need_gpu, say
from parity import check_logits, check_topk
from test_gpu_core import FMTS, make_heads
from test_gpu_linear import torch_bf16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", ["bf16", "block", "row"])
@pytest.mark.parametrize("V,H,R", [(37, 32, 17), (1000, 96, 32), (4133, 1376, 20),
                                   (2051, 4096, 32), (515, 4032, 25), (9000, 1056, 32)])
def test_wide_gemv_parity_and_row_invariance(fmt, V, H, R):
    need_gpu()
    say(f"wide gemv {fmt} V={V} H={H} R={R}")
    w = synth.random_head(V, H, seed=V + H, std=0.02)
    x = synth.random_acts(R, H, seed=R * 7 + H)
    gh, (ow, osc) = make_heads(fmt, w)
    xd = dev_u16(x)
    wide = dh.gemv(gh, xd)
    lo = dh.gemv(gh, xd[:16].contiguous())
    hi = dh.gemv(gh, xd[16:].contiguous())
    one = dh.gemv(gh, xd[R - 1:R].contiguous())
    torch.cuda.synchronize()
    g = host(wide)
    check_logits(g, oracle.gemv(FMTS[fmt][1], ow, osc, x))
    both = np.concatenate([host(lo), host(hi)])
    assert np.array_equal(g.view(np.uint32), both.view(np.uint32))
    assert np.array_equal(g[R - 1].view(np.uint32), host(one)[0].view(np.uint32))


@pytest.mark.parametrize("fmt", ["bf16", "row"])
def test_wide_linear_modes(fmt):
    need_gpu()
    N, K, R = 3001, 4096, 32
    w = synth.random_head(N, K, seed=71, std=0.02)
    x = synth.random_acts(R, K, seed=72)
    res = synth.random_acts(R, N, seed=73, std=0.5)
    gh, (ow, osc) = make_heads(fmt, w)
    xd, rd = dev_u16(x), dev_u16(res)
    f32 = dh.linear(gh, xd, dh.OUT_F32)
    b16 = dh.linear(gh, xd, dh.OUT_BF16)
    add = dh.linear(gh, xd, dh.OUT_ADD_BF16, residual=rd)
    torch.cuda.synchronize()
    gf = host(f32)
    check_logits(gf, oracle.linear(FMTS[fmt][1], ow, osc, x, oracle.MODE_F32), what="linear")
    assert np.array_equal(host(b16).view(np.uint16), torch_bf16(gf))
    resf = (res.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(host(add).view(np.uint16), torch_bf16(resf + gf))


@pytest.mark.parametrize("R,k", [(17, 1), (32, 64), (32, 512)])
def test_wide_draft(R, k):
    need_gpu()
    V, H = 20000, 2048
    w = synth.random_head(V, H, seed=81, std=0.02)
    x = synth.random_acts(R, H, seed=82)
    gh, (ow, osc) = make_heads("block", w)
    out = dh.draft(gh, dev_u16(x), k, keep_logits=True)
    torch.cuda.synchronize()
    glog, ids, vals, dr = (host(out[n]) for n in ("logits", "ids", "vals", "draft"))
    want = oracle.gemv(oracle.FMT_FP8_BLOCK32, ow, osc, x)
    tols = check_logits(glog, want)
    oi, ov = oracle.topk(glog, k)
    assert np.array_equal(ids, oi)
    assert np.array_equal(vals.view(np.uint32), ov.view(np.uint32))
    check_topk(ids, vals, want, k, tols)
    assert np.array_equal(dr, ids[:, 0])


def test_wide_subset_draft():
    need_gpu()
    V, H, n, R, k = 12000, 4096, 4500, 32, 64
    w = synth.random_head(V, H, seed=91, std=0.02)
    x = synth.random_acts(R, H, seed=92)
    gh, _ = make_heads("row", w)
    idmap = synth.token_ids(V, n, seed=93)
    im = dev(idmap)
    sub = dh.gather_rows(gh, im)
    xd = dev_u16(x)
    out = dh.draft_mapped(sub, im, xd, k, keep_logits=True)
    full = dh.gemv(gh, xd)
    torch.cuda.synchronize()
    glog = host(out["logits"])
    assert np.array_equal(glog.view(np.uint32), host(full)[:, idmap].view(np.uint32))
    oi, ov = oracle.topk_mapped(glog, k, idmap)
    assert np.array_equal(host(out["ids"]), oi)


@pytest.mark.parametrize("H", [5120, 7168])
@pytest.mark.parametrize("fmt", ["bf16", "block"])
def test_wide_rows_on_a_wide_head(fmt, H):
    """At H = 5120 a 17..32-row call on an FP8 head runs in one pass (a row-major bf16 head
    takes two 16-row launches), at H = 7168 both take two: parity, and every row the same bits
    as in a 16-row call."""
    need_gpu()
    V, R = 3001, 25
    w = synth.random_head(V, H, seed=95, std=0.02)
    x = synth.random_acts(R, H, seed=96)
    gh, (ow, osc) = make_heads(fmt, w)
    xd = dev_u16(x)
    wide = dh.gemv(gh, xd)
    lo = dh.gemv(gh, xd[:16].contiguous())
    hi = dh.gemv(gh, xd[16:].contiguous())
    res = dev_u16(synth.random_acts(R, V, seed=97, std=0.5))
    add = dh.linear(gh, xd, dh.OUT_ADD_BF16, residual=res)
    torch.cuda.synchronize()
    g = host(wide)
    check_logits(g, oracle.gemv(FMTS[fmt][1], ow, osc, x))
    assert np.array_equal(g.view(np.uint32), np.concatenate([host(lo), host(hi)]).view(np.uint32))
    resf = (host(res).view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(host(add).view(np.uint16), torch_bf16(resf + g))
