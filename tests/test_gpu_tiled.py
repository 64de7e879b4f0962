"""GPU tests of the tiled head layout (DH_TILED) through the C ABI.

 * dh_tile_head writes exactly the layout include/dh.h states (checked against a numpy
   re-arrangement of the row-major bytes, zero padding included);
 * every GEMV form gives bitwise the same results from the tiled head as from the row-major
   one (dh_gemv at 1..32 rows, ragged V and H, all three formats; narrow heads of up to 512
   columns with the draft's cut after them; dh_linear's modes; the
   dh_draft family including the few-tile split of the low-rank down linear), and the tiled
   logits meet the oracle's tolerance;
 * heads that must stay row-major (a rescore's dense head, a gather's source) are refused.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from few_row_vocab_amd import dh
from gpu_util import dev_u16, host, need_gpu, say
from parity import check_logits
from test_gpu_core import FMTS, make_heads

pytestmark = pytest.mark.gpu


def expected_tiled(w, esz):
    """The tiled bytes of a row-major weight (uint8 codes, or uint16 bf16 bits), from the
    layout's statement: block b of tile t holds, for lane l = 16 g + rr, row 16 t + rr's
    elements 64 b + 16 g (+ 8 q for bf16) onward."""
    V, H = w.shape
    T, nkb = -(-V // 16), -(-H // 64)
    p = np.zeros((T * 16, nkb * 64), dtype=w.dtype)
    p[:V, :H] = w
    if esz == 1:
        a = p.reshape(T, 16, nkb, 4, 16).transpose(0, 2, 3, 1, 4)        # t b g rr j
    else:
        a = p.reshape(T, 16, nkb, 4, 2, 8).transpose(0, 2, 4, 3, 1, 5)   # t b q g rr j
    return np.ascontiguousarray(a).reshape(-1).view(np.uint8)


def row_major_bytes(head):
    w = host(head.weight)
    return w.view(np.uint16) if head.format == dh.BF16 else w


SHAPES = [(37, 32), (1000, 96), (4133, 1376), (515, 7168), (2051, 5120), (16, 64)]


@pytest.mark.parametrize("fmt", ["bf16", "block", "row"])
@pytest.mark.parametrize("V,H", SHAPES)
def test_tile_layout(fmt, V, H):
    need_gpu()
    say(f"tile layout {fmt} V={V} H={H}")
    w = synth.random_head(V, H, seed=V * 3 + H, std=0.02)
    gh, _ = make_heads(fmt, w)
    th = dh.tile(gh)
    torch.cuda.synchronize()
    esz = 2 if fmt == "bf16" else 1
    assert th.weight.numel() == dh.tiled_bytes(gh.format, V, H)
    assert th.weight.numel() == -(-V // 16) * -(-H // 64) * 1024 * esz
    assert np.array_equal(host(th.weight), expected_tiled(row_major_bytes(gh), esz))


@pytest.mark.parametrize("fmt", ["bf16", "block", "row"])
@pytest.mark.parametrize("V,H,R", [(37, 32, 1), (1000, 96, 16), (4133, 1376, 5),
                                   (515, 7168, 16), (2051, 5120, 32), (9000, 1056, 20),
                                   (70, 4096, 32), (1, 64, 1), (17, 8192, 3),
                                   (300, 6144, 17)])
def test_tiled_gemv_bit_equal(fmt, V, H, R):
    need_gpu()
    say(f"tiled gemv {fmt} V={V} H={H} R={R}")
    w = synth.random_head(V, H, seed=V + 2 * H, std=0.02)
    x = synth.random_acts(R, H, seed=R + H)
    gh, (ow, osc) = make_heads(fmt, w)
    th = dh.tile(gh)
    xd = dev_u16(x)
    a = host(dh.gemv(gh, xd))
    b = host(dh.gemv(th, xd))
    torch.cuda.synchronize()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    check_logits(b, oracle.gemv(FMTS[fmt][1], ow, osc, x), what="tiled gemv")


# narrow heads (H <= 512: a tile is at most 16 KiB, several workgroups a compute unit): a
# head of one tile (V = 5), H short of a whole 64-column block, tile counts that are not a
# multiple of the grid, heads whose tiles outnumber the row-scale prefetch; the draft's cut
# after them against the row-major head's draft
@pytest.mark.parametrize("fmt", ["bf16", "block", "row"])
@pytest.mark.parametrize("V,H,R", [(5, 512, 16), (100, 32, 3), (4133, 480, 16),
                                   (40000, 512, 1), (40000, 160, 7), (262144, 448, 16)])
def test_tiled_narrow_heads_bit_equal(fmt, V, H, R):
    need_gpu()
    say(f"narrow tiled gemv {fmt} V={V} H={H} R={R}")
    w = synth.random_head(V, H, seed=V + 3 * H, std=0.05)
    x = synth.random_acts(R, H, seed=R + 5 * H)
    gh, (ow, osc) = make_heads(fmt, w)
    th = dh.tile(gh)
    xd = dev_u16(x)
    a = host(dh.gemv(gh, xd))
    b = host(dh.gemv(th, xd))
    torch.cuda.synchronize()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    if V * H <= 25_000_000:
        check_logits(b, oracle.gemv(FMTS[fmt][1], ow, osc, x), what="narrow tiled gemv")
    for k in (1, 64, 512):
        if k <= V:
            c = dh.draft(gh, xd, k, keep_logits=True)
            d = dh.draft(th, xd, k, keep_logits=True)
            torch.cuda.synchronize()
            for n in ("logits", "ids", "vals", "draft"):
                assert host(c[n]).tobytes() == host(d[n]).tobytes(), (k, n)


@pytest.mark.parametrize("R", [16, 32])
@pytest.mark.parametrize("fmt", ["bf16", "row"])
def test_tiled_linear_modes(fmt, R):
    need_gpu()
    N, K = 3001, 2048
    w = synth.random_head(N, K, seed=91, std=0.02)
    x = synth.random_acts(R, K, seed=92)
    res = synth.random_acts(R, N, seed=93, std=0.5)
    gh, _ = make_heads(fmt, w)
    th = dh.tile(gh)
    xd, rd = dev_u16(x), dev_u16(res)
    for mode in (dh.OUT_F32, dh.OUT_BF16, dh.OUT_ADD_BF16):
        r = rd if mode == dh.OUT_ADD_BF16 else None
        a = host(dh.linear(gh, xd, mode, residual=r))
        b = host(dh.linear(th, xd, mode, residual=r))
        assert a.tobytes() == b.tobytes(), f"mode {mode}"


@pytest.mark.parametrize("R,k", [(1, 64), (16, 64), (16, 512), (32, 22)])
def test_tiled_draft_bit_equal(R, k):
    need_gpu()
    V, H = 20000, 2048
    w = synth.random_head(V, H, seed=101, std=0.02)
    x = synth.random_acts(R, H, seed=102)
    gh, _ = make_heads("block", w)
    th = dh.tile(gh)
    xd = dev_u16(x)
    a = dh.draft(gh, xd, k, keep_logits=True)
    b = dh.draft(th, xd, k, keep_logits=True)
    torch.cuda.synchronize()
    for n in ("logits", "ids", "vals", "draft"):
        assert host(a[n]).tobytes() == host(b[n]).tobytes(), n


@pytest.mark.parametrize("R", [16, 32])
def test_tiled_two_stage_and_lowrank(R):
    need_gpu()
    V, H, k, r = 8000, 1024, 128, 256
    w = synth.random_head(V, H, seed=111, std=0.02)
    x = synth.random_acts(R, H, seed=112)
    gr, _ = make_heads("row", w)
    dense = dh.Head(dh.BF16, dev_u16(w))
    xd = dev_u16(x)
    a = dh.draft(gr, xd, k, dense=dense)
    b = dh.draft(dh.tile(gr), xd, k, dense=dense)
    # low rank: a few-tile down linear (r rows: the split over virtual waves, two 16-row
    # column blocks at 32 rows) and the up GEMV
    down = dh.Head(dh.BF16, dev_u16(synth.random_head(r, H, seed=113, std=0.03)))
    up = dh.Head(dh.BF16, dev_u16(synth.random_head(V, r, seed=114, std=0.06)))
    c = dh.draft_lowrank(down, up, xd, k, dense=dense)
    d = dh.draft_lowrank(dh.tile(down), dh.tile(up), xd, k, dense=dense)
    torch.cuda.synchronize()
    for n in ("ids", "vals", "draft", "exact"):
        assert host(a[n]).tobytes() == host(b[n]).tobytes(), n
        assert host(c[n]).tobytes() == host(d[n]).tobytes(), "lowrank " + n


def test_tiled_refusals():
    need_gpu()
    V, H = 300, 256
    w = synth.random_head(V, H, seed=121, std=0.02)
    dense = dh.Head(dh.BF16, dev_u16(w))
    td = dh.tile(dense)
    x = dev_u16(synth.random_acts(2, H, seed=122))
    ids = torch.zeros((2, 4), dtype=torch.int32, device="cuda")
    with pytest.raises(dh.DHError):
        dh.rescore(td, x, ids)
    with pytest.raises(dh.DHError):
        dh.gather_rows(td, torch.arange(10, dtype=torch.int32, device="cuda"))
    with pytest.raises(ValueError):
        dh.tile(td)
    with pytest.raises(dh.DHError):
        dh.draft(td, x, 4, dense=td)


@pytest.mark.slow
@pytest.mark.parametrize("R", [1, 16])
def test_tiled_full_size_bit_equal(R):
    """The benchmarked workload: FP8 E4M3 with E8M0 32x32 blocks, H=5120, V=129280, top-64."""
    need_gpu()
    V, H = 129280, 5120
    say(f"tiled full size R={R}")
    g = torch.Generator(device="cuda").manual_seed(7)
    w = (torch.randn((V, H), device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    codes, scale = dh.quantize(w, dh.FP8_BLOCK32)
    del w
    gh = dh.Head(dh.FP8_BLOCK32, codes, scale)
    th = dh.tile(gh)
    x = torch.randn((R, H), device="cuda", generator=g).to(torch.bfloat16)
    a = dh.draft(gh, x, 64, keep_logits=True)
    b = dh.draft(th, x, 64, keep_logits=True)
    torch.cuda.synchronize()
    for n in ("logits", "ids", "vals", "draft"):
        assert torch.equal(a[n].view(torch.int32) if a[n].dtype == torch.float32 else a[n],
                           b[n].view(torch.int32) if b[n].dtype == torch.float32 else b[n]), n


@pytest.mark.parametrize("fmt", ["block", "row"])
@pytest.mark.parametrize("V,H", SHAPES + [(33, 96), (64, 8192)])
def test_quantize_tiled_equals_tile_of_quantize(fmt, V, H):
    """dh_quantize(format | DH_TILED) writes the same bytes (zero padding included) as
    dh_tile_head of the row-major codes, and the same scale."""
    need_gpu()
    say(f"quantize tiled {fmt} V={V} H={H}")
    w = dev_u16(synth.random_head(V, H, seed=V * 7 + H, std=0.02))
    f = FMTS[fmt][0]
    codes, scale = dh.quantize(w, f)
    ref = dh.tile(dh.Head(f, codes, scale))
    # into buffers pre-filled with 0xAB, so that padding left unwritten would show
    tcodes = torch.full((dh.tiled_bytes(f, V, H),), 0xAB, dtype=torch.uint8, device="cuda")
    tscale = torch.full_like(scale.view(torch.uint8), 0xAB).view(scale.dtype)
    dh._check(dh.lib().dh_quantize(f | dh.TILED, dh._ptr(w), V, H, dh._ptr(tcodes),
                                   dh._ptr(tscale), dh._stream(None)))
    torch.cuda.synchronize()
    assert host(tcodes).tobytes() == host(ref.weight).tobytes()
    assert host(tscale).tobytes() == host(scale).tobytes()
    # the binding's form gives the same bytes
    bcodes, bscale = dh.quantize(w, f | dh.TILED)
    torch.cuda.synchronize()
    assert host(bcodes).tobytes() == host(ref.weight).tobytes()
