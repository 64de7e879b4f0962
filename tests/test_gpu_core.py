"""GPU parity at sizes the oracle finishes in seconds (several tiles, ragged tails): the
quantizers (bit-exact), the GEMV in all formats (logit tolerance), the FP8 widening of every
code and scale byte, top-k on the GPU's own logits (bit-exact against the oracle's top-k),
rescore and the composed draft."""
import numpy as np
import pytest
import torch

import oracle
import synth
from few_row_vocab_amd import dh
from gpu_util import dev, dev_u16, host, need_gpu, say
from parity import check_logits, check_topk

pytestmark = pytest.mark.gpu

FMTS = {"bf16": (dh.BF16, oracle.FMT_BF16), "block": (dh.FP8_BLOCK32, oracle.FMT_FP8_BLOCK32),
        "row": (dh.FP8_ROW, oracle.FMT_FP8_ROW)}


def make_heads(fmt, w):
    """GPU head (quantized on the GPU) and oracle head (quantized by the oracle); the codes
    and scales must agree bit for bit."""
    wd = dev_u16(w)
    if fmt == "bf16":
        return dh.Head(dh.BF16, wd), (w, None)
    f = FMTS[fmt][0]
    codes, scale = dh.quantize(wd, f)
    if fmt == "block":
        oc, os_ = oracle.quant_block32(w)
    else:
        oc, os_ = oracle.quant_row(w)
    torch.cuda.synchronize()
    gc, gs = host(codes), host(scale)
    assert np.array_equal(gc, oc), f"codes differ at {np.count_nonzero(gc != oc)} places"
    assert np.array_equal(gs.view(np.uint8), os_.view(np.uint8)), "scales differ"
    return dh.Head(f, codes, scale), (oc, os_)


@pytest.mark.parametrize("V,H", [(70, 64), (1000, 96), (4133, 1376), (515, 7168), (2051, 5120)])
@pytest.mark.parametrize("fmt", ["block", "row"])
def test_quantize_bit_exact(fmt, V, H):
    need_gpu()
    say(f"quantize {fmt} V={V} H={H}")
    w = synth.random_head(V, H, seed=V + H, std=0.02)
    w[3] = 0                                    # an all-zero row
    make_heads(fmt, w)


def test_quantize_wide_range_bit_exact():
    """Magnitudes over many binades, exact block maxima at 448*2^e, ties of the rounding."""
    need_gpu()
    rng = np.random.default_rng(3)
    V, H = 96, 128
    f = (rng.standard_normal((V, H)) * np.exp2(rng.integers(-30, 30, (V, H)))).astype(np.float32)
    f[0:32, 0:32] = 448.0 * 2.0 ** -3
    f[32, :] = 2.0 ** -9 * 1.5                   # a tie between two codes after scaling
    w = synth.to_bf16_bits(f)
    for fmt in ("block", "row"):
        make_heads(fmt, w)


def test_fp8_widening_every_code_and_scale():
    """Logit v of an identity-like head is decode(code v) * scale exactly: checks the
    in-register E4M3 -> bf16 widening for all 256 codes against the oracle's decoder at
    scale bytes across the exact range."""
    need_gpu()
    V, H = 256, 32
    codes = np.zeros((V, H), np.uint8)
    codes[:, 0] = np.arange(256, dtype=np.uint8)
    x = np.zeros((1, H), np.uint16)
    x[0, 0] = 0x3F80                            # 1.0
    for byte in (10, 60, 100, 120, 127, 128, 140, 200, 246):
        scales = np.full((8, 1), byte, np.uint8)
        scales[3, 0] = 127
        want = oracle.gemv(oracle.FMT_FP8_BLOCK32, codes, scales, x)
        got = host(dh.gemv(dh.Head(dh.FP8_BLOCK32, dev(codes), dev(scales)), dev_u16(x)))
        nan = np.isnan(want)
        assert np.array_equal(nan, np.isnan(got)), byte
        assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32)), byte
    s = np.exp2(np.arange(V) % 7 - 3).astype(np.float32)     # row scales
    want = oracle.gemv(oracle.FMT_FP8_ROW, codes, s, x)
    got = host(dh.gemv(dh.Head(dh.FP8_ROW, dev(codes), dev(s)), dev_u16(x)))
    nan = np.isnan(want)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


@pytest.mark.parametrize("fmt", ["bf16", "block", "row"])
@pytest.mark.parametrize("V,H,R", [(37, 32, 16), (1000, 96, 1), (4133, 1376, 5),
                                   (2051, 5120, 16), (515, 7168, 3), (4096, 256, 1)])
def test_gemv_parity(fmt, V, H, R):
    need_gpu()
    say(f"gemv {fmt} V={V} H={H} R={R}")
    w = synth.random_head(V, H, seed=7 * V + H, std=0.02)
    x = synth.random_acts(R, H, seed=V + 3 * H)
    gh, (ow, osc) = make_heads(fmt, w)
    got = host(dh.gemv(gh, dev_u16(x)))
    want = oracle.gemv(FMTS[fmt][1], ow, osc, x)
    check_logits(got, want)


@pytest.mark.parametrize("fmt", ["bf16", "block"])
def test_gemv_special_rows(fmt):
    """Zero, NaN, +inf and -inf activations: NaN positions and infinities as the oracle."""
    need_gpu()
    V, H = 777, 160
    w = synth.random_head(V, H, seed=11, std=0.02)
    w[5] = 0
    x = synth.random_acts(6, H, seed=12)
    x[1] = 0
    x[2, 17] = 0x7FC0
    x[3, 40] = 0x7F80
    x[4, 99] = 0xFF80
    x[5, 0:32] = synth.to_bf16_bits(np.full(32, 3e38, np.float32))   # overflow to inf
    gh, (ow, osc) = make_heads(fmt, w)
    got = host(dh.gemv(gh, dev_u16(x)))
    want = oracle.gemv(FMTS[fmt][1], ow, osc, x)
    check_logits(got, want)


def _planted(R, V, seed):
    rng = np.random.default_rng(seed)
    rows = []
    kinds = ["normal", "coarse", "nan", "ninf", "equal", "zeros", "sub", "asc", "desc",
             "mixed", "few0", "few1", "few21", "few33", "straddle", "onechunk"]
    for i in range(R):
        kind = kinds[i % len(kinds)]
        if kind == "normal":
            r = rng.standard_normal(V).astype(np.float32)
        elif kind == "coarse":
            r = (rng.integers(-3, 4, V) / 2).astype(np.float32)
        elif kind == "nan":
            r = np.full(V, np.nan, np.float32)
        elif kind == "ninf":
            r = np.full(V, -np.inf, np.float32)
        elif kind == "equal":
            r = np.full(V, 1.5, np.float32)
        elif kind == "zeros":
            r = np.where(rng.random(V) < 0.5, np.float32(0), np.float32(-0.0))
        elif kind == "sub":
            r = (rng.integers(1, 4, V) * 1e-45).astype(np.float32)
        elif kind == "asc":
            r = np.arange(V, dtype=np.float32)
        elif kind == "desc":
            r = -np.arange(V, dtype=np.float32)
        elif kind == "mixed":
            r = rng.standard_normal(V).astype(np.float32)
            r[rng.random(V) < 0.2] = np.nan
            r[rng.random(V) < 0.1] = -np.inf
            r[rng.random(V) < 0.02] = np.inf
        elif kind.startswith("few"):
            m = min(int(kind[3:]), V)
            r = np.full(V, -np.inf, np.float32)
            r[rng.choice(V, m, replace=False)] = rng.standard_normal(m).astype(np.float32)
            r[rng.random(V) < 0.3] = np.nan
        elif kind == "straddle":              # equal values on both sides of chunk edges
            r = rng.standard_normal(V).astype(np.float32) - 10
            for e in range(2048, V, 2048):     # every chunk size is a multiple of 2048
                r[max(0, e - 300):e + 300] = 5.0
        else:                                  # every top value inside one chunk
            r = rng.standard_normal(V).astype(np.float32) - 10
            c0 = (V // 2) // 2048 * 2048
            r[c0:min(V, c0 + 2048)] += 20
        rows.append(r)
    return np.stack(rows)


@pytest.mark.parametrize("V", [70, 4096, 4097, 12345, 163840])
@pytest.mark.parametrize("k", [1, 8, 22, 31, 32, 33, 64, 512])
def test_topk_bit_exact(V, k):
    """Top-k is comparisons only: the GPU must equal the oracle bit for bit on the same
    logits, pads and -0 included."""
    need_gpu()
    if k > V:
        pytest.skip("k > V is refused")
    say(f"topk V={V} k={k}")
    logits = _planted(16, V, seed=V * 1000 + k)
    ids, vals, am = dh.topk(dev(logits), k)
    oi, ov = oracle.topk(logits, k)
    gi, gv = host(ids), host(vals)
    assert np.array_equal(gi, oi)
    assert np.array_equal(gv.view(np.uint32), ov.view(np.uint32))
    assert np.array_equal(host(am), oi[:, 0])


def test_topk_prefix_property():
    """The top-k1 list is the first k1 slots of the top-k2 list (k1 < k2), pads included,
    across every chunk size the top-k picks (k decides it)."""
    need_gpu()
    logits = _planted(16, 40000, seed=77)
    d = dev(logits)
    lists = {k: [host(t) for t in dh.topk(d, k)] for k in (1, 7, 64, 65, 300, 512)}
    ks = sorted(lists)
    for k1, k2 in zip(ks, ks[1:]):
        i1, v1, a1 = lists[k1]
        i2, v2, a2 = lists[k2]
        assert np.array_equal(i1, i2[:, :k1]), (k1, k2)
        assert np.array_equal(v1.view(np.uint32), v2[:, :k1].view(np.uint32)), (k1, k2)
        assert np.array_equal(a1, a2)


@pytest.mark.parametrize("R", [1, 3, 16])
def test_topk_rows(R):
    need_gpu()
    logits = _planted(R, 50000, seed=R)
    ids, vals, am = dh.topk(dev(logits), 100)
    oi, ov = oracle.topk(logits, 100)
    assert np.array_equal(host(ids), oi) and np.array_equal(host(vals).view(np.uint32), ov.view(np.uint32))


def test_rescore_vs_oracle():
    need_gpu()
    V, H, R, ck = 3000, 544, 4, 37
    wd = synth.random_head(V, H, seed=31)
    wd[100] = wd[200]                          # identical rows: an exact tie
    x = synth.random_acts(R, H, seed=32)
    rng = np.random.default_rng(33)
    cand = rng.integers(0, V, (R, ck)).astype(np.int32)
    cand[0, :2] = [200, 100]
    cand[1, 3] = V + 7                          # out of range: NaN, never read
    cand[1, 4] = -2
    cand[2, :] = cand[2, 0]                     # all duplicates
    x[3, 5] = 0x7FC0                            # a NaN row: no eligible candidate
    exact, draft = dh.rescore(dh.Head(dh.BF16, dev_u16(wd)), dev_u16(x), dev(cand))
    oe, od = oracle.rescore(wd, x, cand)
    tols = check_logits(host(exact), oe, what="exact")
    ge, gd = host(exact), host(draft)
    for r in range(R):
        # the winner must be the oracle's wherever its margin exceeds 2 tol
        check_topk_winner(gd[r], oe[r], cand[r], tols[r], od[r])


def check_topk_winner(gdraft, oexact, cand, tol, odraft):
    el = ~np.isnan(oexact) & (oexact != -np.inf)
    if not el.any():
        assert gdraft == 0
        return
    best = oexact[el].max()
    second = np.sort(np.unique(oexact[el]))[-2] if np.unique(oexact[el]).size > 1 else -np.inf
    if best - second > 2 * tol:
        assert gdraft == odraft
    else:
        j = np.nonzero(cand == gdraft)[0]
        assert j.size and oexact[j].max() >= best - 2 * tol


@pytest.mark.parametrize("fmt,two", [("bf16", False), ("block", False), ("row", True),
                                     ("block", True)])
def test_draft_composition_and_parity(fmt, two):
    """dh_draft == dh_topk(dh_gemv) bit for bit; its ids follow the gap rule against the
    oracle; in the two-stage form the rescore follows the oracle run on the GPU's own
    candidate list (the conditional oracle)."""
    need_gpu()
    V, H, R, k = 9000, 1056, 5, 64
    w = synth.random_head(V, H, seed=41, std=0.02)
    x = synth.random_acts(R, H, seed=42)
    gh, (ow, osc) = make_heads(fmt, w)
    dense = dh.Head(dh.BF16, dev_u16(w)) if two else None
    xd = dev_u16(x)
    out = dh.draft(gh, xd, k, dense=dense, keep_logits=True)
    lg = dh.gemv(gh, xd)
    ids, vals, am = dh.topk(lg, k)
    torch.cuda.synchronize()
    assert np.array_equal(host(out["logits"]).view(np.uint32), host(lg).view(np.uint32))
    assert np.array_equal(host(out["ids"]), host(ids))
    assert np.array_equal(host(out["vals"]).view(np.uint32), host(vals).view(np.uint32))
    want = oracle.gemv(FMTS[fmt][1], ow, osc, x)
    tols = check_logits(host(lg), want)
    check_topk(host(out["ids"]), host(out["vals"]), want, k, tols)
    if not two:
        assert np.array_equal(host(out["draft"]), host(am))
        return
    gi, gv = host(out["ids"]), host(out["vals"])
    oe, od = oracle.rescore(w, x, gi, gv > -np.inf)
    etol = check_logits(host(out["exact"]), oe, what="exact")
    for r in range(R):
        check_topk_winner(host(out["draft"])[r], oe[r], gi[r], etol[r], od[r])


@pytest.mark.parametrize("fmt,V,H,R,k", [
    ("block", 37, 32, 16, 1), ("block", 37, 32, 16, 31), ("bf16", 70, 64, 4, 64),
    ("row", 4133, 1376, 5, 22), ("block", 20000, 256, 3, 64), ("bf16", 20000, 256, 16, 8),
    ("block", 50000, 1024, 16, 64), ("row", 9001, 7168, 2, 33)])
def test_draft_equals_topk_of_logits(fmt, V, H, R, k):
    """dh_draft's ids, values and drafts equal dh_topk run on its logits, bit for bit, also
    with exact ties (repeated head rows and coarse activations), a zero row (ids 0..k-1), a
    NaN row (all pads) and +-inf rows."""
    need_gpu()
    rng = np.random.default_rng(V + H + R + k)
    w = synth.random_head(V, H, seed=V + 3, std=0.02)
    for s in range(0, V - 40, max(V // 7, 41)):
        w[s + 1:s + 33] = w[s]                     # 33 identical rows: ties across ids
    x = synth.to_bf16_bits(rng.integers(-2, 3, (R, H)).astype(np.float32) / 8)
    if R > 1:
        x[1] = 0                                   # every logit +-0: ids 0..k-1
    if R > 2:
        x[2, 7] = 0x7FC0                           # NaN: every logit NaN, all pads
    if R > 3:
        x[3, 0:32] = synth.to_bf16_bits(np.full(32, 3e38, np.float32))
    gh, _ = make_heads(fmt, w)
    xd = dev_u16(x)
    say(f"draft vs topk {fmt} V={V} H={H} R={R} k={k}")
    out = dh.draft(gh, xd, k, keep_logits=True)
    ids, vals, am = dh.topk(out["logits"], k)
    lg = dh.gemv(gh, xd)
    torch.cuda.synchronize()
    assert np.array_equal(host(out["logits"]).view(np.uint32), host(lg).view(np.uint32))
    assert np.array_equal(host(out["ids"]), host(ids))
    assert np.array_equal(host(out["vals"]).view(np.uint32), host(vals).view(np.uint32))
    assert np.array_equal(host(out["draft"]), host(am))
    if R > 2:
        assert np.all(host(out["ids"])[2] == 0) and np.all(host(out["vals"])[2] == -np.inf)
    if R > 1:
        assert np.array_equal(host(out["ids"])[1], np.arange(k))
