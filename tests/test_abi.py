"""The C-ABI library on the CPU: it loads, exports every symbol include/dh.h declares, and
refuses bad arguments on the host before touching any pointer (no GPU needed: refused calls
never reach the HIP runtime, so host buffers stand in for device buffers and must come back
untouched)."""
import ctypes
import os
import re

import numpy as np
import pytest

from few_row_vocab_amd import dh

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "dh.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dh_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = dh.lib()
    names = declared_functions()
    assert set(names) >= {"dh_gemv", "dh_topk", "dh_rescore", "dh_rescore_sync", "dh_draft",
                          "dh_quantize", "dh_linear_ws", "dh_linear_workspace_bytes",
                          "dh_workspace_bytes", "dh_status_string", "dh_gather_rows",
                          "dh_topk_mapped", "dh_draft_mapped", "dh_linear",
                          "dh_draft_lowrank", "dh_topk_softmax", "dh_sample"}
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for s in range(6):
        assert dh.status_string(s) and dh.status_string(s) != "unknown status"
    assert dh.status_string(99) == "unknown status"


def test_workspace_bytes_limits():
    assert dh.workspace_bytes(16, 163840, 512) > 16 * 163840 * 4
    assert dh.workspace_bytes(0, 1000, 8) == 0
    assert dh.workspace_bytes(33, 1000, 8) == 0
    assert dh.workspace_bytes(32, 1000, 8) > dh.workspace_bytes(16, 1000, 8)
    assert dh.workspace_bytes(1, 1000, 0) == 0
    assert dh.workspace_bytes(1, 1000, 513) == 0
    assert dh.workspace_bytes(1, 10, 11) == 0
    assert dh.workspace_bytes(1, dh.MAX_VOCAB + 1, 8) == 0
    # grows with each size
    assert dh.workspace_bytes(2, 5000, 8) > dh.workspace_bytes(1, 5000, 8)
    assert dh.workspace_bytes(1, 5000, 64) >= dh.workspace_bytes(1, 5000, 8)
    assert dh.workspace_bytes(1, 129280, 512) > dh.workspace_bytes(1, 129280, 8)


@pytest.fixture
def no_device():
    # These calls hand host memory to the library as if it were device memory; they are
    # only safe because every one of them is refused before a launch.  Where a GPU is
    # visible, the GPU suite repeats the refusals on real device buffers instead.
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-buffer refusal tests run only where no GPU is visible")


class HostBuf:
    """Aligned host memory standing in for device buffers in refusal tests."""

    def __init__(self, nbytes, fill=0xAB, align=256):
        self.raw = np.full(nbytes + align, fill, np.uint8)
        off = (-self.raw.ctypes.data) % align
        self.a = self.raw[off:off + nbytes]
        self.fill = fill

    @property
    def p(self):
        return ctypes.c_void_p(self.a.ctypes.data)

    def untouched(self):
        return bool(np.all(self.a == self.fill))


def head(fmt, V, H, w, s=None):
    return dh._Head(fmt, V, H, w.a.ctypes.data if w else None,
                    s.a.ctypes.data if s else None)


def call_gemv(h, x, rows, out):
    return dh.lib().dh_gemv(ctypes.byref(h), x.p if x else None, rows,
                            out.p if out else None, None)


def test_gemv_refusals_leave_outputs_untouched(no_device):
    V, H = 100, 64
    w, s, x, out = HostBuf(V * H), HostBuf(4 * H // 32), HostBuf(16 * H * 2), HostBuf(16 * V * 4)
    ok = head(dh.FP8_BLOCK32, V, H, w, s)
    cases = [
        (ok, x, 0, out, 1), (ok, x, 33, out, 2), (ok, None, 1, out, 1), (ok, x, 1, None, 1),
        (head(7, V, H, w, s), x, 1, out, 1),                       # bad format
        (head(dh.FP8_BLOCK32, V, 48, w, s), x, 1, out, 1),         # H % 32
        (head(dh.FP8_BLOCK32, V, 32800, w, s), x, 1, out, 2),      # H > 32768
        (head(dh.FP8_BLOCK32, 0, H, w, s), x, 1, out, 1),          # V < 1
        (head(dh.FP8_BLOCK32, V, H, w, None), x, 1, out, 1),       # missing scale
        (head(dh.BF16, V, H, w, s), x, 1, out, 1),                 # bf16 with a scale
        (head(dh.FP8_BLOCK32, V, H, None, s), x, 1, out, 1),       # null weight
    ]
    for h, xx, rows, o, want in cases:
        assert call_gemv(h, xx, rows, o) == want, (h.format, h.vocab, h.hidden, rows)
    # misaligned weight / activations
    h = dh._Head(dh.FP8_BLOCK32, V, H, w.a.ctypes.data + 4, s.a.ctypes.data)
    assert call_gemv(h, x, 1, out) == 1
    xm = ctypes.c_void_p(x.a.ctypes.data + 2)
    assert dh.lib().dh_gemv(ctypes.byref(ok), xm, 1, out.p, None) == 1
    # output overlapping the weights
    assert dh.lib().dh_gemv(ctypes.byref(ok), x.p, 1, w.p, None) == 1
    assert out.untouched()


def test_topk_refusals_leave_outputs_untouched(no_device):
    R, V, k = 2, 1000, 8
    lg, ids, vals, am = HostBuf(R * V * 4), HostBuf(R * k * 4), HostBuf(R * k * 4), HostBuf(R * 4)
    ws = HostBuf(dh.workspace_bytes(R, V, k))
    L = dh.lib()

    def call(rows=R, vocab=V, kk=k, wsb=None, wsp=None, logits=None, i=None):
        wsb = ws.a.size if wsb is None else wsb
        return L.dh_topk((logits or lg).p, rows, vocab, kk, (i or ids).p, vals.p, am.p,
                         ws.p if wsp is None else wsp, wsb, None)

    assert call(kk=0) == 1
    assert call(kk=513) == 2
    assert call(kk=V + 1) == 1
    assert call(rows=0) == 1 and call(rows=33) == 2
    assert call(vocab=dh.MAX_VOCAB + 1) == 2
    assert call(wsb=64) == 3
    assert call(wsp=ctypes.c_void_p(ws.a.ctypes.data + 16)) == 3      # misaligned workspace
    assert call(i=vals) == 1                                            # ids overlap vals
    assert ids.untouched() and vals.untouched() and am.untouched()


def test_rescore_and_draft_refusals(no_device):
    R, V, H, k = 2, 600, 64, 16
    w, wd, s = HostBuf(V * H), HostBuf(V * H * 2), HostBuf(V * 4)
    x, ids, vals, ex, dr = (HostBuf(R * H * 2), HostBuf(R * k * 4), HostBuf(R * k * 4),
                            HostBuf(R * k * 4), HostBuf(R * 4))
    ws = HostBuf(dh.workspace_bytes(R, V, k))
    L = dh.lib()
    dense = head(dh.BF16, V, H, wd)
    stage1 = head(dh.FP8_ROW, V, H, w, s)
    # rescore: dense head must be bf16; cand_k range
    assert L.dh_rescore(ctypes.byref(stage1), x.p, R, ids.p, k, ex.p, dr.p, None) == 1
    assert L.dh_rescore(ctypes.byref(dense), x.p, R, ids.p, 0, ex.p, dr.p, None) == 1
    assert L.dh_rescore(ctypes.byref(dense), x.p, R, ids.p, 513, ex.p, dr.p, None) == 2
    assert L.dh_rescore(ctypes.byref(dense), x.p, R, ids.p, k, ids.p, dr.p, None) == 1

    lg = HostBuf(R * V * 4)

    def draft(h=stage1, d=dense, rows=R, kk=k, exact=ex, wsb=None, logits=None, drf=dr):
        return L.dh_draft(ctypes.byref(h), ctypes.byref(d) if d else None, x.p, rows, kk,
                          ids.p, vals.p, drf.p, exact.p if exact else None,
                          logits.p if logits else None, ws.p,
                          ws.a.size if wsb is None else wsb, None)

    assert draft(exact=vals) == 1                       # exact overlaps the stage-1 values
    assert draft(exact=w) == 1                          # exact overlaps the stage-1 weight
    assert draft(exact=s) == 1                          # exact overlaps the stage-1 scale
    assert draft(exact=lg, logits=lg) == 1              # exact overlaps the logits
    assert draft(drf=lg, logits=lg) == 1                # draft overlaps the logits
    assert draft(exact=ws) == 1                         # exact inside the workspace
    assert draft(drf=ws) == 1                           # draft inside the workspace
    assert draft(d=None, exact=None, drf=w) == 1        # one-stage draft over the weight
    assert draft(exact=None) == 1                       # two-stage needs `exact`
    assert draft(d=None) == 1                           # one-stage must not pass `exact`
    assert draft(d=head(dh.BF16, V - 1, H, wd)) == 1   # dense head of another size
    assert draft(d=stage1) == 1                         # dense head not bf16
    assert draft(kk=513) == 2
    assert draft(wsb=100) == 3
    assert draft(rows=33) == 2
    for b in (ids, vals, ex, dr, lg):
        assert b.untouched()


def test_rescore_sync_refusals(no_device):
    """dh_rescore_sync refuses what dh_rescore refuses, and a missing, misaligned or
    overlapping sync buffer, on the host."""
    R, V, H, k = 2, 600, 64, 16
    wd, x, ids, ex, dr = (HostBuf(V * H * 2), HostBuf(R * H * 2), HostBuf(R * k * 4),
                          HostBuf(R * k * 4), HostBuf(R * 4))
    sync = HostBuf(dh.RESCORE_SYNC_BYTES)
    big = HostBuf(dh.RESCORE_SYNC_BYTES + 4096)
    L = dh.lib()
    dense = head(dh.BF16, V, H, wd)

    def call(d=dense, rows=R, kk=k, exact=ex, sp=None):
        return L.dh_rescore_sync(ctypes.byref(d), x.p, rows, ids.p, kk, exact.p, dr.p,
                                 sync.p if sp is None else sp, None)

    assert call(d=head(dh.FP8_ROW, V, H, wd, HostBuf(V * 4))) == 1   # dense head not bf16
    assert call(d=head(dh.BF16 | dh.TILED, V, H, wd)) == 1            # tiled dense head
    assert call(kk=0) == 1 and call(kk=513) == 2
    assert call(rows=0) == 1 and call(rows=33) == 2
    assert call(exact=ids) == 1                                        # exact overlaps ids
    assert L.dh_rescore_sync(ctypes.byref(dense), x.p, R, ids.p, k, ex.p, dr.p, None,
                             None) == 1                                # no sync buffer
    assert call(sp=ctypes.c_void_p(big.a.ctypes.data + 16)) == 1       # misaligned
    assert call(sp=ex.p) == 1                                          # sync overlaps exact
    assert call(sp=dr.p) == 1                                          # sync overlaps draft
    assert call(sp=wd.p) == 1                                          # sync in the weight
    assert call(sp=x.p) == 1                                           # sync overlaps x
    for b in (ids, ex, dr, sync, big):
        assert b.untouched()


def test_quantize_refusals(no_device):
    L = dh.lib()
    w, c, s = HostBuf(64 * 64 * 2), HostBuf(64 * 64), HostBuf(256)
    assert L.dh_quantize(dh.BF16, w.p, 64, 64, c.p, s.p, None) == 1
    assert L.dh_quantize(dh.FP8_ROW, w.p, 64, 48, c.p, s.p, None) == 1
    assert L.dh_quantize(dh.FP8_ROW, w.p, 0, 64, c.p, s.p, None) == 1
    assert L.dh_quantize(dh.FP8_ROW, w.p, 64, 64, None, s.p, None) == 1
    assert L.dh_quantize(dh.FP8_BLOCK32, w.p, 64, 64, w.p, s.p, None) == 1   # overlap
    assert L.dh_quantize(dh.BF16 | dh.TILED, w.p, 64, 64, c.p, s.p, None) == 1
    assert L.dh_quantize(dh.FP8_ROW | 64, w.p, 64, 64, c.p, s.p, None) == 1  # unknown bits
    cm = ctypes.c_void_p(c.a.ctypes.data + 8)                                # tiled: 16-B
    assert L.dh_quantize(dh.FP8_ROW | dh.TILED, w.p, 64, 64, cm, s.p, None) == 1
    assert c.untouched() and s.untouched()


def test_subset_refusals(no_device):
    """dh_gather_rows, dh_topk_mapped and dh_draft_mapped refuse on the host."""
    L = dh.lib()
    V, H, n = 600, 64, 40
    w, wd, s, blk = HostBuf(V * H), HostBuf(V * H * 2), HostBuf(V * 4), HostBuf(1024)
    ids_in = HostBuf(n * 4, fill=0)
    ow, os_ = HostBuf(n * H * 2), HostBuf(n * 4)
    row = head(dh.FP8_ROW, V, H, w, s)
    bf = head(dh.BF16, V, H, wd)
    g = lambda h, i=ids_in, nn=n, o=ow, sc=os_: L.dh_gather_rows(
        ctypes.byref(h), i.p if i else None, nn, o.p if o else None, sc.p if sc else None, None)
    assert g(head(dh.FP8_BLOCK32, V, H, w, blk)) == 2     # 32x32 blocks cannot be split
    assert g(row, nn=0) == 1
    assert g(row, i=None) == 1 and g(row, o=None) == 1
    assert g(row, sc=None) == 1                           # per-row FP8 needs the scale out
    assert g(bf, sc=os_) == 1                             # bf16 has no scale
    assert g(row, o=w) == 1                               # output overlaps the head
    assert g(row, sc=ids_in) == 1                         # scale out overlaps the ids
    assert L.dh_gather_rows(ctypes.byref(row), ids_in.p, n,
                            ctypes.c_void_p(ow.a.ctypes.data + 8), os_.p, None) == 1
    assert ow.untouched() and os_.untouched()

    R, k = 2, 8
    lg, ti, tv, am = HostBuf(R * n * 4), HostBuf(R * k * 4), HostBuf(R * k * 4), HostBuf(R * 4)
    idmap = HostBuf(n * 4, fill=0)
    ws = HostBuf(dh.workspace_bytes(R, n, k))
    t = lambda m=idmap, i=ti, kk=k: L.dh_topk_mapped(lg.p, R, n, kk, m.p if m else None,
                                                     i.p, tv.p, am.p, ws.p, ws.a.size, None)
    assert t(m=None) == 1
    assert t(kk=n + 1) == 1
    assert t(i=idmap) == 1                                # ids overlap the map
    assert ti.untouched() and tv.untouched() and am.untouched()

    sub = head(dh.FP8_ROW, n, H, HostBuf(n * H), HostBuf(n * 4))
    x, ex, dr = HostBuf(R * H * 2), HostBuf(R * k * 4), HostBuf(R * 4)
    dws = HostBuf(dh.workspace_bytes(R, n, k))

    def d(m=idmap, dense=bf, exact=ex, i=ti):
        return L.dh_draft_mapped(ctypes.byref(sub), m.p if m else None,
                                 ctypes.byref(dense) if dense else None, x.p, R, k, i.p,
                                 tv.p, dr.p, exact.p if exact else None, None, dws.p,
                                 dws.a.size, None)

    assert d(m=None) == 1
    assert d(dense=head(dh.BF16, V, 96, HostBuf(V * 96 * 2))) == 1   # other width
    assert d(dense=row) == 1                                         # dense not bf16
    assert d(exact=None) == 1
    assert d(i=idmap) == 1                                           # ids overlap the map
    assert d(dense=None, exact=idmap) == 1
    for b in (ti, tv, ex, dr):
        assert b.untouched()


def test_linear_refusals(no_device):
    L = dh.lib()
    N, K, R = 96, 64, 2
    w, s, x = HostBuf(N * K), HostBuf(N * 4), HostBuf(R * K * 2)
    out, res = HostBuf(R * N * 4), HostBuf(R * N * 2)
    h = head(dh.FP8_ROW, N, K, w, s)
    c = lambda mode, r=res, o=out, rows=R: L.dh_linear(ctypes.byref(h), x.p, rows, mode,
                                                       r.p if r else None, o.p, None)
    assert c(3, r=None) == 1                       # unknown mode
    assert c(dh.OUT_ADD_BF16, r=None) == 1         # the add mode needs a residual
    assert c(dh.OUT_BF16) == 1                     # only the add mode takes one
    assert c(dh.OUT_F32, r=None, rows=33) == 2
    assert c(dh.OUT_F32, r=None, o=w) == 1         # out overlaps the weight
    part = ctypes.c_void_p(out.a.ctypes.data + 2)
    assert L.dh_linear(ctypes.byref(h), x.p, R, dh.OUT_ADD_BF16, out.p, part, None) == 1
    assert L.dh_linear(ctypes.byref(h), x.p, R, dh.OUT_F32, None, part, None) == 1  # misaligned
    assert out.untouched() and res.untouched()


def test_lowrank_refusals(no_device):
    L = dh.lib()
    H, rk, V, R, k = 128, 64, 700, 2, 8
    wd, wu, wdense = HostBuf(rk * H * 2), HostBuf(V * rk * 2), HostBuf(V * H * 2)
    x, t = HostBuf(R * H * 2), HostBuf(R * rk * 2)
    ids, vals, ex, dr = HostBuf(R * k * 4), HostBuf(R * k * 4), HostBuf(R * k * 4), HostBuf(R * 4)
    ws = HostBuf(dh.workspace_bytes(R, V, k))
    down, up = head(dh.BF16, rk, H, wd), head(dh.BF16, V, rk, wu)
    dense = head(dh.BF16, V, H, wdense)

    def c(dn=down, u=up, d=dense, tt=t, exact=ex):
        return L.dh_draft_lowrank(ctypes.byref(dn) if dn else None, ctypes.byref(u),
                                  ctypes.byref(d) if d else None, x.p, R, k,
                                  tt.p if tt else None, ids.p, vals.p, dr.p,
                                  exact.p if exact else None, None, ws.p, ws.a.size, None)

    assert c(dn=None) == 1
    assert c(tt=None) == 1                                     # t is required
    assert c(u=head(dh.BF16, V, 96, wu)) == 1                  # up width != rank
    assert c(d=head(dh.BF16, V, rk, wdense)) == 1              # dense width != H
    assert c(tt=x) == 1                                        # t overlaps x
    assert c(tt=ids) == 1                                      # t overlaps an output
    assert c(d=None) == 1                                      # one stage with `exact`
    for b in (ids, vals, ex, dr, t):
        assert b.untouched()


def test_topk_softmax_refusals(no_device):
    L = dh.lib()
    R, V, k = 2, 1000, 8
    lg, ids, vals = HostBuf(R * V * 4), HostBuf(R * k * 4), HostBuf(R * k * 4)
    probs, lse = HostBuf(R * k * 4), HostBuf(R * 4)
    ws = HostBuf(dh.workspace_bytes(R, V, k))
    c = lambda pr=probs, ls=lse: L.dh_topk_softmax(lg.p, R, V, k, ids.p, vals.p, None,
                                                   pr.p if pr else None, ls.p if ls else None,
                                                   ws.p, ws.a.size, None)
    assert c(pr=None) == 1 and c(ls=None) == 1
    assert c(ls=ids) == 1                       # lse overlaps ids
    assert c(pr=vals) == 1                      # probs overlap vals
    assert c(ls=probs) == 1                     # lse overlaps probs
    assert c(ls=lg) == 1                        # lse overlaps the logits
    for b in (ids, vals, probs, lse):
        assert b.untouched()


def test_sample_refusals(no_device):
    L = dh.lib()
    R, k = 2, 8
    ids, vals, pos, tok, kept = (HostBuf(R * k * 4), HostBuf(R * k * 4), HostBuf(R * 8),
                                 HostBuf(R * 4), HostBuf(R * 4))
    c = lambda T=1.0, p=1.0, m=0.0, rows=R, kk=k, t=tok: L.dh_sample(
        ids.p, vals.p, rows, kk, T, p, m, 1, pos.p, t.p, kept.p, None)
    assert c(T=-1.0) == 1 and c(T=float("nan")) == 1 and c(T=float("inf")) == 1
    assert c(p=0.0) == 1 and c(p=1.01) == 1 and c(m=-0.5) == 1 and c(m=2.0) == 1
    assert c(rows=0) == 1 and c(rows=33) == 2 and c(kk=0) == 1 and c(kk=513) == 2
    assert c(t=ids) == 1                          # token overlaps the candidates
    assert tok.untouched() and kept.untouched()


def test_tiled_bytes():
    # ceil(V/16) tiles x ceil(H/64) blocks x 1 KiB x bytes per element
    assert dh.tiled_bytes(dh.FP8_BLOCK32, 129280, 5120) == 8080 * 80 * 1024
    assert dh.tiled_bytes(dh.FP8_BLOCK32 | dh.TILED, 129280, 5120) == 8080 * 80 * 1024
    assert dh.tiled_bytes(dh.BF16, 129280, 5120) == 8080 * 80 * 2048
    assert dh.tiled_bytes(dh.FP8_ROW, 37, 96) == 3 * 2 * 1024
    assert dh.tiled_bytes(dh.BF16, 16, 32) == 1 * 1 * 2048
    assert dh.tiled_bytes(dh.FP8_ROW, 0, 96) == 0
    assert dh.tiled_bytes(dh.FP8_ROW, 100, 48) == 0
    assert dh.tiled_bytes(dh.FP8_ROW, 100, 32800) == 0
    assert dh.tiled_bytes(7, 100, 64) == 0
    assert dh.tiled_bytes(dh.FP8_ROW | 32, 100, 64) == 0


def test_tiled_refusals(no_device):
    V, H = 100, 64
    w, s, x, out = HostBuf(V * H), HostBuf(4 * H // 32), HostBuf(16 * H * 2), HostBuf(16 * V * 4)
    tb = dh.tiled_bytes(dh.FP8_BLOCK32, V, H)
    tw = HostBuf(tb)
    L = dh.lib()
    ok = head(dh.FP8_BLOCK32, V, H, w, s)
    # dh_tile_head: a tiled source, a null or misaligned target, a target over the head
    assert L.dh_tile_head(ctypes.byref(head(dh.FP8_BLOCK32 | dh.TILED, V, H, w, s)), tw.p,
                          None) == 1
    assert L.dh_tile_head(ctypes.byref(ok), None, None) == 1
    assert L.dh_tile_head(ctypes.byref(ok), ctypes.c_void_p(tw.a.ctypes.data + 8), None) == 1
    assert L.dh_tile_head(ctypes.byref(ok), w.p, None) == 1
    assert L.dh_tile_head(ctypes.byref(head(dh.FP8_BLOCK32, V, 48, w, s)), tw.p, None) == 1
    assert tw.untouched()
    # a tiled head: unknown modifier bits, output over the tiled weight, a tiled dense head
    th = head(dh.FP8_BLOCK32 | dh.TILED, V, H, tw, s)
    assert call_gemv(head(dh.FP8_BLOCK32 | 64, V, H, tw, s), x, 1, out) == 1
    assert call_gemv(th, x, 1, tw) == 1
    assert out.untouched()
    dense_t = head(dh.BF16 | dh.TILED, V, H, HostBuf(dh.tiled_bytes(dh.BF16, V, H)))
    ids, exact, draft = HostBuf(4 * 4), HostBuf(4 * 4), HostBuf(4)
    assert L.dh_rescore(ctypes.byref(dense_t), x.p, 1, ids.p, 4, exact.p, draft.p, None) == 1
    assert exact.untouched() and draft.untouched()
    gw = HostBuf(10 * H * 2)
    assert L.dh_gather_rows(ctypes.byref(dense_t), ids.p, 4, gw.p, None, None) == 1
    assert gw.untouched()


def test_stream_read_refusals(no_device):
    buf, sink = HostBuf(8192), HostBuf(dh.STREAM_SINK_WORDS * 4)
    L = dh.lib()
    assert L.dh_stream_read(None, 8192, sink.p, None) == 1
    assert L.dh_stream_read(buf.p, 8192, None, None) == 1
    assert L.dh_stream_read(buf.p, 0, sink.p, None) == 1
    assert L.dh_stream_read(buf.p, 4100, sink.p, None) == 1
    assert L.dh_stream_read(ctypes.c_void_p(buf.a.ctypes.data + 4), 4096, sink.p, None) == 1
    assert L.dh_stream_read(buf.p, 8192, ctypes.c_void_p(buf.a.ctypes.data + 4096), None) == 1
    assert sink.untouched() and buf.untouched()


def test_draft_noalloc_refusals(no_device):
    """dh_draft_noalloc refuses, before any launch, what dh_draft refuses and sizes beyond its
    fixed scratch (DH_ERR_SCRATCH, 5)."""
    L = dh.lib()
    R, V, H, k = 2, 600, 64, 16
    w, s = HostBuf(V * H), HostBuf(((V + 31) // 32) * (H // 32))
    x, ids, vals, dr = HostBuf(R * H * 2), HostBuf(R * k * 4), HostBuf(R * k * 4), HostBuf(R * 4)
    hd = head(dh.FP8_BLOCK32, V, H, w, s)

    def call(h=hd, rows=R, kk=k, drf=dr, logits=None):
        return L.dh_draft_noalloc(ctypes.byref(h), None, x.p, rows, kk, ids.p, vals.p, drf.p,
                                  None, logits.p if logits else None, None)

    assert call(rows=0) == 1
    assert call(rows=33) == 2
    assert call(kk=513) == 2
    assert call(drf=vals) == 1                                 # draft overlaps vals
    assert call(drf=w) == 1                                    # draft over the weight
    # 32 rows of 200,000 logits (25.6 MB) do not fit the 16 MiB scratch without `logits`
    big = head(dh.FP8_BLOCK32, 200000, H, w, s)
    assert call(h=big, rows=32) == 5
    assert dh.workspace_bytes(32, 200000, k) > dh.NOALLOC_SCRATCH_BYTES
    for b in (ids, vals, dr):
        assert b.untouched()


def test_linear_ws_refusals(no_device):
    """dh_linear_ws refuses what dh_linear refuses, and a missing, short, misaligned or
    overlapping workspace, on the host."""
    N, K, R = 300, 16384, 2
    L = dh.lib()
    nb = L.dh_linear_workspace_bytes(R, N, K)
    assert nb >= 2 * R * N * 4 and nb % 256 == 0
    assert L.dh_linear_workspace_bytes(0, N, K) == 0 and L.dh_linear_workspace_bytes(33, N, K) == 0
    assert L.dh_linear_workspace_bytes(R, N, 48) == 0 and L.dh_linear_workspace_bytes(R, 0, K) == 0
    assert L.dh_linear_workspace_bytes(R, N, 32768 + 32) == 0
    w, s, x, out = HostBuf(N * K), HostBuf(N * 4), HostBuf(R * K * 2), HostBuf(R * N * 4)
    ws = HostBuf(nb + 512)
    h = head(dh.FP8_ROW, N, K, w, s)

    def call(mode=dh.OUT_F32, wsp=None, wsb=None, o=out):
        return L.dh_linear_ws(ctypes.byref(h), x.p, R, mode, None, o.p,
                              ws.p if wsp is None else wsp, nb if wsb is None else wsb, None)

    assert call(mode=3) == 1                                            # unknown mode
    assert L.dh_linear_ws(ctypes.byref(h), x.p, R, dh.OUT_F32, None, out.p, None, nb,
                          None) == 3                                    # no workspace
    assert call(wsb=nb - 256) == 3                                      # short
    assert call(wsp=ctypes.c_void_p(ws.a.ctypes.data + 64)) == 3        # misaligned
    assert call(o=ws) == 1                                              # output in the workspace
    assert call(wsp=w.p, wsb=N * K) == 1                                # over the weight
    for b in (w, s, x, out, ws):
        assert b.untouched()
