"""GPU tests: dh_draft's top-k equals dh_topk's on the draft's own logits, bit for bit (ids,
values, argmax), and the oracle's under the gap rule, on inputs that stress a row's top-k
being concentrated in one place:
 * random heads, one to 32 rows, k from 1 to 64, all formats, tiled and row-major heads,
   ragged vocabularies;
 * planted heads whose best rows crowd into one 16-row tile (one GEMV workgroup, one top-k
   chunk holds up to 16 of a row's top-k): distinct values and exact ties (lower id first),
   and a row with fewer eligible logits than k;
 * the two-stage and the mapped (subset) drafts;
 * for dh_draft's fused top-k (up to 16 rows: each GEMV workgroup leaves a short cut of its
   logits, a per-row merge checks it and reads back the chunks whose cut may be short): rows
   of exact ties everywhere (every cut empty, the whole row read back in passes), runs of
   consecutive best ids spanning many tiles (one chunk per tile holding 16 of the k), and
   k = 512 over 16 rows.
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


@pytest.mark.parametrize("k", [1, 64, 512])
def test_draft_topk_all_tied_rows(k):
    """Rows of zero activations: every logit is a zero (ties everywhere), so the top-k is ids
    0..k-1; every GEMV workgroup's cut is empty and the merge reads the row back in passes
    (70,001 logits: several passes of 16,384)."""
    need_gpu()
    V, H = 70001, 256
    say(f"all-tied rows k={k}")
    w = synth.random_head(V, H, seed=151, std=0.02)
    x = np.stack([np.zeros(H, np.uint16), synth.random_acts(1, H, seed=152)[0],
                  np.zeros(H, np.uint16)])
    gh = dh.Head(dh.BF16, dev_u16(w))
    out = draft_vs_topk(gh, dev_u16(x), k, tile=True)
    ids, vals = host(out["ids"]), host(out["vals"])
    for r in (0, 2):
        assert ids[r].tolist() == list(range(k))
        assert np.all(vals[r] == 0)
    want = oracle.gemv(oracle.FMT_BF16, w, None, x)
    tols = check_logits(host(out["logits"]), want)
    check_topk(ids, vals, want, k, tols)


def clustered_head(V, H, lo, n, seed):
    """A head whose rows lo..lo+n-1 are the activation row `base` scaled by 1 + j/256 (in bf16):
    for x = base they are the row's n largest logits, over n / 16 tiles."""
    w = synth.random_head(V, H, seed=seed, std=0.02).copy()
    base = synth.random_acts(1, H, seed=seed + 1)[0]
    scale = 1.0 + np.arange(n, dtype=np.float32) / 256
    w[lo:lo + n] = synth.to_bf16_bits(synth.bf16_bits_to_f32(base)[None, :] * scale[:, None])
    return w, base


@pytest.mark.parametrize("k,n", [(64, 64), (64, 200), (512, 600)])
def test_draft_topk_clustered_ids(k, n):
    """The k best ids of a row are consecutive and span many 16-row tiles, so many GEMV
    workgroups each hold 16 of them, more than their cuts keep: the merge reads those
    workgroups' logits back and still returns the exact top-k, all from the planted run."""
    need_gpu()
    V, H, lo = 60000, 512, 1000
    say(f"clustered ids k={k} n={n}")
    w, base = clustered_head(V, H, lo, n, seed=161 + k)
    x = np.stack([base, synth.random_acts(1, H, seed=162)[0]])
    gh = dh.Head(dh.BF16, dev_u16(w))
    out = draft_vs_topk(gh, dev_u16(x), k, tile=True)
    want = oracle.gemv(oracle.FMT_BF16, w, None, x)
    tols = check_logits(host(out["logits"]), want)
    check_topk(host(out["ids"]), host(out["vals"]), want, k, tols)
    # the planted rows' logits dwarf the others' (their order within the run is the oracle
    # check's: bf16 rounding of base * (1 + j/256) ties or swaps neighbours)
    top = host(out["ids"])[0]
    assert np.all((top >= lo) & (top < lo + n))
    if k == n:
        assert sorted(top.tolist()) == list(range(lo, lo + n))


@pytest.mark.parametrize("fmt", ["block", "row"])
def test_draft_topk_512_sixteen_rows(fmt):
    need_gpu()
    V, H, R, k = 129280, 1024, 16, 512
    say(f"top-512 of 16 rows {fmt}")
    w = synth.random_head(V, H, seed=171, std=0.02)
    x = synth.random_acts(R, H, seed=172)
    gh, (ow, osc) = make_heads(fmt, w)
    out = draft_vs_topk(gh, dev_u16(x), k, tile=True)
    want = oracle.gemv(FMTS[fmt][1], ow, osc, x)
    tols = check_logits(host(out["logits"]), want)
    check_topk(host(out["ids"]), host(out["vals"]), want, k, tols)


@pytest.mark.parametrize("tile", [False, True])
@pytest.mark.parametrize("k", [17, 64, 512])
def test_draft_topk_32_rows(tile, k):
    """32 rows (one GEMV launch of two 16-row column blocks, then the top-k's own cut pass
    and merge) of a clustered head: the first 8 along its planted run (their best keys crowd
    a few chunks, whose cuts are short), the next 8 zero (every logit tied, every cut
    empty), the rest random."""
    need_gpu()
    V, H, lo, n = 60000, 512, 1000, 600
    say(f"32 rows tile={tile} k={k}")
    w, base = clustered_head(V, H, lo, n, seed=181 + k)
    x = np.concatenate([np.repeat(base[None, :], 8, axis=0), np.zeros((8, H), np.uint16),
                        synth.random_acts(16, H, seed=182)])
    gh = dh.Head(dh.BF16, dev_u16(w))
    out = draft_vs_topk(gh, dev_u16(x), k, tile=tile)
    want = oracle.gemv(oracle.FMT_BF16, w, None, x)
    tols = check_logits(host(out["logits"]), want)
    check_topk(host(out["ids"]), host(out["vals"]), want, k, tols)
    ids = host(out["ids"])
    for r in range(8, 16):
        assert ids[r].tolist() == list(range(k))


@pytest.mark.parametrize("fmt", ["block", "bf16"])
def test_draft_topk_two_launch_rows(fmt):
    """More than 16 rows of a head too wide for one launch (H = 7168; a row-major bf16 head
    at H = 5120) take two GEMV launches (rows 0..15, then the rest), then the top-k."""
    need_gpu()
    V, H, R, k = 9000, 7168 if fmt == "block" else 5120, 20, 64
    say(f"two-launch rows {fmt} H={H}")
    w = synth.random_head(V, H, seed=191, std=0.02)
    x = synth.random_acts(R, H, seed=192)
    gh, (ow, osc) = make_heads(fmt, w)
    out = draft_vs_topk(gh, dev_u16(x), k, tile=(fmt == "block"))
    want = oracle.gemv(FMTS[fmt][1], ow, osc, x)
    tols = check_logits(host(out["logits"]), want)
    check_topk(host(out["ids"]), host(out["vals"]), want, k, tols)
