"""GPU tests: dh_draft's top-k equals dh_topk's on the draft's own logits, bit for bit (ids,
values, argmax), and the oracle's under the gap rule, on inputs that stress a row's top-k
being concentrated in one place:
 * random heads, one to 32 rows, k from 1 to 64, all formats, tiled and row-major heads,
   ragged vocabularies;
 * planted heads whose best rows crowd into one 16-row tile (one GEMV workgroup, one top-k
   chunk holds up to 16 of a row's top-k): distinct values and exact ties (lower id first),
   and a row with fewer eligible logits than k;
 * the two-stage and the mapped (subset) drafts.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from few_row_vocab_amd import dh
from gpu_util import dev_u16, host, need_gpu, say
from parity import check_logits, check_topk
from test_gpu_core import FMTS, make_heads

pytestmark = pytest.mark.gpu


def draft_vs_topk(head, xd, k, tile=False):
    """dh_draft's outputs and dh_topk's on the draft's own logits; asserts bit equality."""
    h = dh.tile(head) if tile else head
    out = dh.draft(h, xd, k, keep_logits=True)
    ids, vals, am = dh.topk(out["logits"], k)
    torch.cuda.synchronize()
    assert np.array_equal(host(out["ids"]), host(ids))
    assert host(out["vals"]).tobytes() == host(vals).tobytes()
    assert np.array_equal(host(out["draft"]), host(am))
    return out


@pytest.mark.parametrize("fmt", ["bf16", "block", "row"])
@pytest.mark.parametrize("V,H,R,k", [(20000, 1024, 1, 1), (20000, 1024, 1, 64),
                                     (4133, 1376, 16, 9), (4133, 1376, 16, 64),
                                     (130001, 256, 5, 5), (130001, 256, 5, 22),
                                     (9000, 2048, 32, 8), (9000, 2048, 32, 64)])
def test_draft_topk_random(fmt, V, H, R, k):
    need_gpu()
    say(f"list top-k {fmt} V={V} H={H} R={R} k={k}")
    w = synth.random_head(V, H, seed=V + H + k, std=0.02)
    x = synth.random_acts(R, H, seed=R + 3 * k)
    gh, (ow, osc) = make_heads(fmt, w)
    out = draft_vs_topk(gh, dev_u16(x), k, tile=(k % 2 == 0))
    want = oracle.gemv(FMTS[fmt][1], ow, osc, x)
    tols = check_logits(host(out["logits"]), want)
    check_topk(host(out["ids"]), host(out["vals"]), want, k, tols)


def crowded_head(V, H, seed, tie):
    """A head whose rows 32..47 (one 16-row tile, so one GEMV workgroup) are the activation
    row `base` scaled by 1 + j/64 (tie: all equal to base): for x = base they hold the row's 16
    largest logits, distinct (largest at row 47) or tied exactly (the lower id first)."""
    w = synth.random_head(V, H, seed=seed, std=0.02).copy()
    base = synth.random_acts(1, H, seed=seed + 1)[0]
    scale = np.ones(16, np.float32) if tie else 1.0 + np.arange(16, dtype=np.float32) / 64
    w[32:48] = synth.to_bf16_bits(synth.bf16_bits_to_f32(base)[None, :] * scale[:, None])
    return w, base


@pytest.mark.parametrize("tie", [False, True])
@pytest.mark.parametrize("k", [9, 16, 17, 33, 64])
def test_draft_topk_crowded_tile(tie, k):
    need_gpu()
    V, H = 50000, 512
    say(f"crowded tile tie={tie} k={k}")
    w, base = crowded_head(V, H, seed=131 + k, tie=tie)
    x = np.stack([base, base, synth.random_acts(1, H, seed=5)[0]])
    gh = dh.Head(dh.BF16, dev_u16(w))
    out = draft_vs_topk(gh, dev_u16(x), k, tile=True)
    want = oracle.gemv(oracle.FMT_BF16, w, None, x)
    tols = check_logits(host(out["logits"]), want)
    check_topk(host(out["ids"]), host(out["vals"]), want, k, tols)
    ids = host(out["ids"])
    lead = min(k, 16)
    order = list(range(32, 48)) if tie else list(range(47, 31, -1))
    for r in (0, 1):                   # rows 0 and 1 point along the crowded tile
        assert ids[r][:lead].tolist() == order[:lead]


def test_draft_topk_fewer_eligible_than_k():
    """A row whose logits are NaN except a crowded tile's 16: fewer eligible than k, so the
    pads (id 0, -inf) follow the 16."""
    need_gpu()
    V, H, k = 8000, 256, 64
    w = np.zeros((V, H), np.uint16)
    nan16 = np.uint16(0x7FC0)
    w[:, 0] = nan16                                   # every logit NaN ...
    w[32:48, 0] = synth.to_bf16_bits(np.float32([1.0]))[0]
    w[32:48, 1] = synth.to_bf16_bits(np.arange(16, dtype=np.float32) / 16)
    x = np.zeros((1, H), np.uint16)
    x[0, 0] = synth.to_bf16_bits(np.float32([1.0]))[0]
    x[0, 1] = synth.to_bf16_bits(np.float32([1.0]))[0]
    gh = dh.Head(dh.BF16, dev_u16(w))
    out = draft_vs_topk(gh, dev_u16(x), k)
    ids, vals = host(out["ids"])[0], host(out["vals"])[0]
    assert ids[:16].tolist() == list(range(47, 31, -1))   # 1 + j/16, largest j first
    assert np.all(ids[16:] == 0) and np.all(np.isneginf(vals[16:]))
    want = oracle.gemv(oracle.FMT_BF16, w, None, x)
    oi, ov = oracle.topk(want.astype(np.float32), k)
    assert np.array_equal(ids, oi[0])


@pytest.mark.parametrize("k", [8, 64])
def test_draft_topk_two_stage_and_mapped(k):
    need_gpu()
    V, H, R = 30000, 1024, 16
    w = synth.random_head(V, H, seed=141, std=0.02)
    x = synth.random_acts(R, H, seed=142)
    gr, _ = make_heads("row", w)
    xd = dev_u16(x)
    dense = dh.Head(dh.BF16, dev_u16(w))
    two = dh.draft(dh.tile(gr), xd, k, dense=dense, keep_logits=True)
    ids, vals, _ = dh.topk(two["logits"], k)
    torch.cuda.synchronize()
    assert np.array_equal(host(two["ids"]), host(ids))
    assert host(two["vals"]).tobytes() == host(vals).tobytes()
    # the subset head: the mapped merge reports vocabulary ids
    im = torch.from_numpy(synth.token_ids(V, 7000, seed=143)).cuda()
    sub = dh.gather_rows(gr, im)
    mo = dh.draft_mapped(dh.tile(sub), im, xd, k, keep_logits=True)
    mi, mv, ma = dh.topk_mapped(mo["logits"], k, im)
    torch.cuda.synchronize()
    assert np.array_equal(host(mo["ids"]), host(mi))
    assert host(mo["vals"]).tobytes() == host(mv).tobytes()
    assert np.array_equal(host(mo["draft"]), host(ma))
