"""GPU parity of dh_linear (the draft head's own linears through the few-row GEMV) against
the oracle's O14, through the C ABI, for the three weight formats and the three output modes.

 * fp32 mode: within the logit tolerance of the oracle, and bit-identical to dh_gemv;
 * bf16 modes: bit-identical to the GPU's own fp32 sums rounded on the host (torch's
   float32 -> bfloat16, round to nearest even; for the add mode after a float32 add of the
   residual), and within tol_r + one bf16 ulp of the oracle's single rounding, where tol_r
   is the fp32 logit tolerance of the row;
 * the add mode in place (out == residual) equals the add mode into a fresh buffer.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from few_row_vocab_amd import dh
from gpu_util import dev_u16, host, need_gpu, say
from parity import check_logits, row_tol
from test_gpu_core import FMTS, make_heads

pytestmark = pytest.mark.gpu


def torch_bf16(f32):
    t = torch.from_numpy(np.ascontiguousarray(f32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_f32(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32)


def check_bf16(gpu_bits, orc_bits, orc_pre, what):
    """|gpu - oracle| <= tol_r + ulp_bf16 (the larger magnitude's), NaN/inf as the oracle."""
    g, o = bf16_f32(gpu_bits), bf16_f32(orc_bits)
    for r in range(o.shape[0]):
        tol = row_tol(orc_pre[r])
        fin = np.isfinite(o[r])
        assert np.array_equal(np.isnan(g[r]), np.isnan(o[r])), f"{what} row {r}: NaN"
        assert np.array_equal(np.isinf(g[r]), np.isinf(o[r])), f"{what} row {r}: inf"
        mag = np.maximum(np.abs(g[r][fin]), np.abs(o[r][fin])).astype(np.float64)
        ulp = np.exp2(np.floor(np.log2(np.maximum(mag, 2.0**-126))) - 7)
        err = np.abs(g[r][fin].astype(np.float64) - o[r][fin])
        assert np.all(err <= tol + ulp), f"{what} row {r}: {float((err - tol - ulp).max()):.3e}"


def _check_modes(gh, x, res, of, ow, osc):
    """dh_linear's three modes on head gh against the oracle's O14 (and the bf16 modes against
    the GPU's own fp32 sums rounded on the host); returns the GPU outputs."""
    xd, rd = dev_u16(x), dev_u16(res)
    f32 = dh.linear(gh, xd, dh.OUT_F32)
    b16 = dh.linear(gh, xd, dh.OUT_BF16)
    add = dh.linear(gh, xd, dh.OUT_ADD_BF16, residual=rd)
    inplace = rd.clone()
    dh.linear(gh, xd, dh.OUT_ADD_BF16, residual=inplace, out=inplace)
    logits = dh.gemv(gh, xd)
    torch.cuda.synchronize()
    gf, gb, ga, gi = host(f32), host(b16).view(np.uint16), host(add).view(np.uint16), \
        host(inplace).view(np.uint16)
    assert np.array_equal(gf.view(np.uint32), host(logits).view(np.uint32))
    want = oracle.linear(of, ow, osc, x, oracle.MODE_F32)
    check_logits(gf, want, what="linear f32")
    # the bf16 modes round the GPU's own fp32 sums
    assert np.array_equal(gb, torch_bf16(gf))
    assert np.array_equal(ga, torch_bf16(bf16_f32(res) + gf))
    assert np.array_equal(gi, ga)
    check_bf16(gb, oracle.linear(of, ow, osc, x, oracle.MODE_BF16), want, "linear bf16")
    pre = bf16_f32(res).astype(np.float64) + want
    check_bf16(ga, oracle.linear(of, ow, osc, x, oracle.MODE_ADD_BF16, res), pre,
               "linear add")
    return gf, gb, ga


@pytest.mark.parametrize("fmt", ["bf16", "block", "row"])
@pytest.mark.parametrize("N,K,R", [(37, 32, 16), (1000, 96, 1), (4133, 1376, 5),
                                   (5120, 5120, 16), (2051, 8192, 3)])
def test_linear_modes(fmt, N, K, R):
    need_gpu()
    say(f"linear {fmt} N={N} K={K} R={R}")
    w = synth.random_head(N, K, seed=N + K, std=0.02)
    x = synth.random_acts(R, K, seed=R + K)
    res = synth.random_acts(R, N, seed=N + R, std=0.5)
    gh, (ow, osc) = make_heads(fmt, w)
    _check_modes(gh, x, res, FMTS[fmt][1], ow, osc)


@pytest.mark.parametrize("fmt", ["bf16", "block", "row"])
@pytest.mark.parametrize("N,K,R", [(2051, 16384, 3), (5120, 18432, 16), (300, 32768, 32),
                                   (77, 8256, 1)])
def test_linear_wide(fmt, N, K, R):
    """Inputs wider than 8192 (a w2 whose input is the FFN width): the GEMV streams the
    columns in chunks of 8192.  All three modes against the oracle, and the tiled head bit
    for bit equal to the row-major one (both take the same chunks and virtual waves)."""
    need_gpu()
    say(f"wide linear {fmt} N={N} K={K} R={R}")
    w = synth.random_head(N, K, seed=N + K, std=0.02)
    x = synth.random_acts(R, K, seed=R + K)
    res = synth.random_acts(R, N, seed=N + R, std=0.5)
    gh, (ow, osc) = make_heads(fmt, w)
    of = FMTS[fmt][1]
    gf, gb, ga = _check_modes(gh, x, res, of, ow, osc)
    th = dh.tile(gh)
    xd, rd = dev_u16(x), dev_u16(res)
    tf = dh.linear(th, xd, dh.OUT_F32)
    tb = dh.linear(th, xd, dh.OUT_BF16)
    ta = dh.linear(th, xd, dh.OUT_ADD_BF16, residual=rd)
    torch.cuda.synchronize()
    assert np.array_equal(host(tf).view(np.uint32), gf.view(np.uint32))
    assert np.array_equal(host(tb).view(np.uint16), gb)
    assert np.array_equal(host(ta).view(np.uint16), ga)
    # a row's sums do not depend on how many rows share the call
    one = dh.linear(th, xd[R - 1:R].contiguous(), dh.OUT_F32)
    torch.cuda.synchronize()
    assert np.array_equal(host(one)[0].view(np.uint32), gf[R - 1].view(np.uint32))


def test_linear_refusals_on_device():
    need_gpu()
    N, K, R = 64, 64, 2
    w = synth.random_head(N, K, seed=5, std=0.02)
    gh, _ = make_heads("row", w)
    xd = dev_u16(synth.random_acts(R, K, seed=6))
    out = torch.zeros((R, N), dtype=torch.int16, device="cuda")
    with pytest.raises(dh.DHError):
        dh.linear(gh, xd, 3, out=out)                                  # unknown mode
    with pytest.raises(dh.DHError):
        dh.linear(gh, xd, dh.OUT_ADD_BF16, out=out)                    # add without residual
    with pytest.raises(dh.DHError):
        dh.linear(gh, xd, dh.OUT_BF16, residual=out.clone(), out=out)  # residual without add
    big = torch.zeros((R * N + 8,), dtype=torch.int16, device="cuda")
    with pytest.raises(dh.DHError):                                    # partial overlap
        dh.linear(gh, xd, dh.OUT_ADD_BF16, residual=big[8:].view(R, N), out=big[:R * N].view(R, N))
    torch.cuda.synchronize()
    assert not host(out).any() and not host(big).any()


@pytest.mark.parametrize("fmt", ["bf16", "block", "row"])
@pytest.mark.parametrize("N,K,R", [(2051, 16384, 3), (5120, 18432, 16), (300, 32768, 16),
                                   (77, 8256, 1), (320, 5120, 5), (40000, 9024, 2),
                                   (300, 32768, 20)])
def test_linear_ws_equals_linear(fmt, N, K, R):
    """dh_linear_ws gives dh_linear's bits in every mode, on both layouts: with K above 8192
    and few output tiles the column chunks of every tile run at once (partials in the
    workspace, summed in chunk order); with K up to 8192 and few tiles, the split by 64-column
    parts; otherwise (many tiles, or more than 16 rows) the workspace goes unused."""
    need_gpu()
    say(f"linear_ws {fmt} N={N} K={K} R={R}")
    w = synth.random_head(N, K, seed=N + 3 * K, std=0.02)
    x = dev_u16(synth.random_acts(R, K, seed=R + 5 * K))
    res = dev_u16(synth.random_acts(R, N, seed=N + R + 1, std=0.5))
    gh, _ = make_heads(fmt, w)
    ws = dh.linear_workspace(R, N, K)
    ws.fill_(0xFF)                                   # stale contents must not matter
    for head in (gh, dh.tile(gh)):
        for mode in (dh.OUT_F32, dh.OUT_BF16, dh.OUT_ADD_BF16):
            r = res if mode == dh.OUT_ADD_BF16 else None
            a = dh.linear(head, x, mode, residual=r)
            b = dh.linear(head, x, mode, residual=r, ws=ws)
            torch.cuda.synchronize()
            assert np.array_equal(host(a).view(np.uint8), host(b).view(np.uint8)), mode
    # in place: out == residual
    acc = res.clone()
    dh.linear(gh, x, dh.OUT_ADD_BF16, residual=acc, out=acc, ws=ws)
    want = dh.linear(gh, x, dh.OUT_ADD_BF16, residual=res)
    torch.cuda.synchronize()
    assert np.array_equal(host(acc).view(np.uint16), host(want).view(np.uint16))


def test_linear_ws_refusals_on_device():
    need_gpu()
    N, K, R = 300, 16384, 2
    w = synth.random_head(N, K, seed=15, std=0.02)
    gh, _ = make_heads("row", w)
    xd = dev_u16(synth.random_acts(R, K, seed=16))
    out = torch.zeros((R, N), dtype=torch.float32, device="cuda")
    nb = dh.linear_workspace_bytes(R, N, K)
    assert nb >= 2 * R * N * 4                       # two column chunks of partials
    with pytest.raises(dh.DHError):                  # short
        dh.linear(gh, xd, dh.OUT_F32, out=out, ws=torch.empty(nb - 256, dtype=torch.uint8,
                                                               device="cuda"))
    big = torch.zeros(nb + R * N * 4 + 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(dh.DHError):                  # the output inside the workspace
        dh.linear(gh, xd, dh.OUT_F32, out=big[:R * N * 4].view(torch.float32).view(R, N),
                  ws=big[:nb])
    torch.cuda.synchronize()
    assert not host(out).any()
