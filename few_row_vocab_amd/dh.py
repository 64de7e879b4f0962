"""Python binding of libdh.so (include/dh.h): argument marshalling only.

Every step of the projection runs in the library's HIP kernels; torch provides device
buffers and the current stream.  There is no fallback: if libdh.so is missing or a call is
refused, this module raises.
"""
import ctypes
import functools
import os
from dataclasses import dataclass
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdh.so")

BF16 = 0
FP8_BLOCK32 = 1
FP8_ROW = 2
FORMATS = {"bf16": BF16, "fp8_block32": FP8_BLOCK32, "fp8_row": FP8_ROW}
TILED = 16   # layout modifier: the weight tiled for the GEMV (see tile())

OUT_F32 = 0
OUT_BF16 = 1
OUT_ADD_BF16 = 2

MAX_ROWS = 32
MAX_HIDDEN_WIDE = 5120   # 4096 for a row-major bf16 head
MAX_K = 512
MAX_HIDDEN = 32768
MAX_VOCAB = 262144
RESCORE_SYNC_BYTES = MAX_ROWS * 2 * 256   # DH_RESCORE_SYNC_BYTES

STATUS = {0: "DH_OK", 1: "DH_ERR_INVALID", 2: "DH_ERR_UNSUPPORTED", 3: "DH_ERR_WORKSPACE",
          4: "DH_ERR_DEVICE", 5: "DH_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 16 << 20   # the fixed scratch of dh_draft_noalloc


class DHError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class _Head(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("vocab", ctypes.c_int64),
                ("hidden", ctypes.c_int64), ("weight", ctypes.c_void_p),
                ("scale", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libdh.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python few_row_vocab_amd/build.py` (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        c = ctypes
        hp, vp, i32, i64, sz = c.POINTER(_Head), c.c_void_p, c.c_int32, c.c_int64, c.c_size_t
        L.dh_gemv.argtypes = [hp, vp, i32, vp, vp]
        L.dh_topk.argtypes = [vp, i32, i64, i32, vp, vp, vp, vp, sz, vp]
        L.dh_rescore.argtypes = [hp, vp, i32, vp, i32, vp, vp, vp]
        L.dh_rescore_sync.argtypes = [hp, vp, i32, vp, i32, vp, vp, vp, vp]
        L.dh_draft.argtypes = [hp, hp, vp, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.dh_draft_noalloc.argtypes = [hp, hp, vp, i32, i32, vp, vp, vp, vp, vp, vp]
        L.dh_quantize.argtypes = [i32, vp, i64, i64, vp, vp, vp]
        L.dh_gather_rows.argtypes = [hp, vp, i64, vp, vp, vp]
        L.dh_linear.argtypes = [hp, vp, i32, i32, vp, vp, vp]
        L.dh_linear_ws.argtypes = [hp, vp, i32, i32, vp, vp, vp, sz, vp]
        L.dh_linear_workspace_bytes.argtypes = [i32, i64, i64]
        L.dh_linear_workspace_bytes.restype = sz
        L.dh_topk_softmax.argtypes = [vp, i32, i64, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.dh_sample.argtypes = [vp, vp, i32, i32, c.c_double, c.c_double, c.c_double,
                                c.c_uint64, vp, vp, vp, vp]
        L.dh_draft_lowrank.argtypes = [hp, hp, hp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                       sz, vp]
        L.dh_topk_mapped.argtypes = [vp, i32, i64, i32, vp, vp, vp, vp, vp, sz, vp]
        L.dh_draft_mapped.argtypes = [hp, vp, hp, vp, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.dh_tile_head.argtypes = [hp, vp, vp]
        L.dh_stream_read.argtypes = [vp, sz, vp, vp]
        L.dh_tiled_bytes.argtypes = [i32, i64, i64]
        L.dh_tiled_bytes.restype = sz
        L.dh_workspace_bytes.argtypes = [i32, i64, i32]
        L.dh_workspace_bytes.restype = sz
        L.dh_status_string.argtypes = [i32]
        L.dh_status_string.restype = c.c_char_p
        for f in (L.dh_gemv, L.dh_topk, L.dh_rescore, L.dh_rescore_sync, L.dh_draft,
                  L.dh_draft_noalloc,
                  L.dh_quantize,
                  L.dh_gather_rows, L.dh_topk_mapped, L.dh_draft_mapped, L.dh_linear,
                  L.dh_linear_ws,
                  L.dh_draft_lowrank, L.dh_topk_softmax, L.dh_sample, L.dh_tile_head,
                  L.dh_stream_read):
            f.restype = i32
        _lib = L
    return _lib


def _on_stream(fn):
    """Run a binding call with `stream` (when given) as torch's current stream, so that the
    outputs and any temporary workspace it allocates belong to the stream the library
    launches on: the caching allocator then cannot hand a freed temporary to other work
    while the kernels on that stream still use it."""
    @functools.wraps(fn)
    def call(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, stream=None, **kw)
        with torch.cuda.stream(stream):
            return fn(*args, stream=stream, **kw)
    return call


def _check(status):
    if status != 0:
        raise DHError(status, lib().dh_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _want(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")


def _shaped(t, shape, dtypes, name):
    """A caller's tensor must match what the library will read or write through its pointer:
    the C ABI takes bare pointers and cannot check sizes itself."""
    if t is None:
        return None
    dtypes = dtypes if isinstance(dtypes, tuple) else (dtypes,)
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: expected {' or '.join(map(str, dtypes))}, got {t.dtype}")
    _want(t, t.dtype, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


BF16_BITS = (torch.bfloat16, torch.int16)


def _ws_bytes(ws):
    if ws.dtype != torch.uint8:
        raise TypeError("workspace: expected a uint8 tensor")
    _want(ws, torch.uint8, "workspace")
    return ws.numel()


def _bits16(t):
    """bf16 tensors are passed as their bit patterns."""
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@dataclass
class Head:
    """A vocabulary head: weight [V][H] (bf16, or uint8 E4M3 codes) and its scale (None,
    uint8 E8M0 [ceil(V/32)][H/32], or float32 [V]).  A tiled head (format | TILED, made by
    tile()) holds its weight as a flat uint8 buffer of tiled_bytes() and its (V, H) in
    `shape`."""
    format: int
    weight: torch.Tensor
    scale: Optional[torch.Tensor] = None
    shape: Optional[tuple] = None

    @property
    def tiled(self):
        return bool(self.format & TILED)

    @property
    def base_format(self):
        return self.format & ~TILED

    @property
    def vocab(self):
        return self.shape[0] if self.tiled else self.weight.shape[0]

    @property
    def hidden(self):
        return self.shape[1] if self.tiled else self.weight.shape[1]

    def _c(self):
        w = self.weight
        fmt = self.base_format
        if self.tiled:
            if self.shape is None or len(self.shape) != 2:
                raise ValueError("a tiled head needs shape (V, H)")
            V, H = (int(d) for d in self.shape)
            if w.dtype != torch.uint8 or w.dim() != 1:
                raise TypeError("tiled head: weight must be a flat uint8 buffer")
            _want(w, torch.uint8, "weight")
            if w.numel() != tiled_bytes(self.format, V, H):
                raise ValueError(f"tiled head: weight must hold {tiled_bytes(self.format, V, H)} "
                                 f"bytes, has {w.numel()}")
        else:
            if fmt == BF16:
                if w.dtype not in (torch.bfloat16, torch.int16):
                    raise TypeError("bf16 head: weight must be bfloat16 (or its int16 bits)")
            elif w.dtype != torch.uint8:
                raise TypeError("FP8 head: weight must be uint8 E4M3 codes")
            _want(w, w.dtype, "weight")
            if w.dim() != 2:
                raise ValueError("weight: expected [V][H]")
            V, H = w.shape
        if fmt == FP8_ROW:
            _shaped(self.scale, (V,), torch.float32, "scale")
        elif fmt == FP8_BLOCK32:
            _shaped(self.scale, ((V + 31) // 32, H // 32), torch.uint8, "scale")
        elif self.scale is not None:
            raise ValueError("a bf16 head has no scale")
        return _Head(self.format, V, H, w.data_ptr(),
                     None if self.scale is None else self.scale.data_ptr())


def tiled_bytes(format, vocab, hidden):
    """Bytes of a tiled weight (dh_tiled_bytes); 0 for sizes the library refuses."""
    return int(lib().dh_tiled_bytes(format, vocab, hidden))


@_on_stream
def tile(head: Head, stream=None):
    """The tiled copy of a row-major head (dh_tile_head): same format | TILED, same scale;
    the GEMV forms give bitwise the same results from it and stream it faster."""
    if head.tiled:
        raise ValueError("the head is already tiled")
    n = tiled_bytes(head.format, head.vocab, head.hidden)
    if n == 0:
        raise DHError(2, "sizes outside the library's limits")
    out = torch.empty((n,), dtype=torch.uint8, device=head.weight.device)
    h = head._c()
    _check(lib().dh_tile_head(ctypes.byref(h), _ptr(out), _stream(stream)))
    return Head(head.format | TILED, out, head.scale, (head.vocab, head.hidden))


def workspace_bytes(rows, vocab, k):
    return int(lib().dh_workspace_bytes(rows, vocab, k))


def workspace(rows, vocab, k, device="cuda"):
    n = workspace_bytes(rows, vocab, k)
    if n == 0:
        raise DHError(2, "sizes outside the library's limits")
    return torch.empty(n, dtype=torch.uint8, device=device)


@_on_stream
def gemv(head: Head, x, logits=None, stream=None):
    """logits [R][V] fp32 = x [R][H] (bf16) times the head."""
    R = x.shape[0]
    _shaped(x, (R, head.hidden), BF16_BITS, "x")
    if logits is None:
        logits = torch.empty((R, head.vocab), dtype=torch.float32, device=x.device)
    _shaped(logits, (R, head.vocab), torch.float32, "logits")
    h = head._c()
    _check(lib().dh_gemv(ctypes.byref(h), _ptr(x), R, _ptr(logits), _stream(stream)))
    return logits


@_on_stream
def linear(w: Head, x, mode=OUT_F32, residual=None, out=None, ws=None, stream=None):
    """out [R][N] = x [R][K] (bf16) times the linear w [N][K]: float32 (OUT_F32), bf16
    (OUT_BF16) or bf16 of residual + the sum (OUT_ADD_BF16; out may be residual).  With `ws`
    (linear_workspace(R, N, K)): dh_linear_ws, the same bits, faster for few output rows."""
    R = x.shape[0]
    _shaped(x, (R, w.hidden), BF16_BITS, "x")
    if out is None:
        dt = torch.float32 if mode == OUT_F32 else torch.int16
        out = torch.empty((R, w.vocab), dtype=dt, device=x.device)
    _shaped(out, (R, w.vocab), torch.float32 if mode == OUT_F32 else BF16_BITS, "out")
    _shaped(residual, (R, w.vocab), BF16_BITS, "residual")
    h = w._c()
    if ws is not None:
        _check(lib().dh_linear_ws(ctypes.byref(h), _ptr(x), R, mode, _ptr(residual), _ptr(out),
                                  _ptr(ws), _ws_bytes(ws), _stream(stream)))
    else:
        _check(lib().dh_linear(ctypes.byref(h), _ptr(x), R, mode, _ptr(residual), _ptr(out),
                               _stream(stream)))
    return out


def linear_workspace_bytes(rows, n, k):
    return int(lib().dh_linear_workspace_bytes(rows, n, k))


def linear_workspace(rows, n, k, device="cuda"):
    """A workspace for linear(..., ws=) over `rows` rows of a linear with n outputs and k
    inputs."""
    nb = linear_workspace_bytes(rows, n, k)
    if nb == 0:
        raise DHError(2, "sizes outside the library's limits")
    return torch.empty(nb, dtype=torch.uint8, device=device)


@_on_stream
def _topk_call(logits, k, idmap, ws, ids, vals, argmax, with_argmax, stream):
    _want(logits, torch.float32, "logits")
    R, V = logits.shape
    dev = logits.device
    ids = torch.empty((R, k), dtype=torch.int32, device=dev) if ids is None else ids
    vals = torch.empty((R, k), dtype=torch.float32, device=dev) if vals is None else vals
    if with_argmax and argmax is None:
        argmax = torch.empty((R,), dtype=torch.int32, device=dev)
    _shaped(ids, (R, k), torch.int32, "ids")
    _shaped(vals, (R, k), torch.float32, "vals")
    _shaped(argmax, (R,), torch.int32, "argmax")
    ws = workspace(R, V, k, dev) if ws is None else ws
    if idmap is None:
        st = lib().dh_topk(_ptr(logits), R, V, k, _ptr(ids), _ptr(vals), _ptr(argmax),
                           _ptr(ws), _ws_bytes(ws), _stream(stream))
    else:
        _want(idmap, torch.int32, "idmap")
        if idmap.numel() != V:
            raise ValueError(f"idmap: expected {V} ids, got {idmap.numel()}")
        st = lib().dh_topk_mapped(_ptr(logits), R, V, k, _ptr(idmap), _ptr(ids), _ptr(vals),
                                  _ptr(argmax), _ptr(ws), _ws_bytes(ws), _stream(stream))
    _check(st)
    return ids, vals, argmax


def topk(logits, k, ws=None, ids=None, vals=None, argmax=None, with_argmax=True,
         stream=None):
    """(ids int32 [R][k], vals fp32 [R][k], argmax int32 [R] or None)."""
    return _topk_call(logits, k, None, ws, ids, vals, argmax, with_argmax, stream=stream)


def topk_mapped(logits, k, idmap, ws=None, ids=None, vals=None, argmax=None,
                with_argmax=True, stream=None):
    """topk over a subset head's logits; ids and argmax are vocabulary ids idmap[j]."""
    return _topk_call(logits, k, idmap, ws, ids, vals, argmax, with_argmax, stream=stream)


@_on_stream
def topk_softmax(logits, k, ws=None, with_argmax=True, stream=None, out=None):
    """(ids, vals, argmax, probs fp32 [R][k], lse fp32 [R]): dh_topk plus each row's softmax
    statistics (probs[:, 0] is the top-1's confidence).  `out`: a dict of preallocated
    outputs (ids, vals, probs, lse, argmax), any of them."""
    _want(logits, torch.float32, "logits")
    R, V = logits.shape
    dev = logits.device
    o = {} if out is None else out
    ids = o.get("ids")
    ids = torch.empty((R, k), dtype=torch.int32, device=dev) if ids is None else ids
    vals = o.get("vals")
    vals = torch.empty((R, k), dtype=torch.float32, device=dev) if vals is None else vals
    probs = o.get("probs")
    probs = torch.empty((R, k), dtype=torch.float32, device=dev) if probs is None else probs
    lse = o.get("lse")
    lse = torch.empty((R,), dtype=torch.float32, device=dev) if lse is None else lse
    argmax = o.get("argmax")
    if argmax is None and with_argmax:
        argmax = torch.empty((R,), dtype=torch.int32, device=dev)
    _shaped(ids, (R, k), torch.int32, "ids")
    _shaped(vals, (R, k), torch.float32, "vals")
    _shaped(probs, (R, k), torch.float32, "probs")
    _shaped(lse, (R,), torch.float32, "lse")
    _shaped(argmax, (R,), torch.int32, "argmax")
    ws = workspace(R, V, k, dev) if ws is None else ws
    _check(lib().dh_topk_softmax(_ptr(logits), R, V, k, _ptr(ids), _ptr(vals), _ptr(argmax),
                                 _ptr(probs), _ptr(lse), _ptr(ws), _ws_bytes(ws),
                                 _stream(stream)))
    return ids, vals, argmax, probs, lse


@_on_stream
def sample(ids, vals, positions, temperature=1.0, top_p=1.0, min_p=0.0, seed=0,
           with_kept=True, token=None, kept=None, stream=None):
    """dh_sample: (token int32 [R], kept int32 [R] or None) keyed by seed, positions (int64
    [R]) and the candidates' token ids."""
    _want(ids, torch.int32, "ids")
    R, k = ids.shape
    _shaped(vals, (R, k), torch.float32, "vals")
    _shaped(positions, (R,), torch.int64, "positions")
    if token is None:
        token = torch.empty((R,), dtype=torch.int32, device=ids.device)
    if kept is None and with_kept:
        kept = torch.empty((R,), dtype=torch.int32, device=ids.device)
    _shaped(token, (R,), torch.int32, "token")
    _shaped(kept, (R,), torch.int32, "kept")
    _check(lib().dh_sample(_ptr(ids), _ptr(vals), R, k, float(temperature), float(top_p),
                           float(min_p), int(seed) & (2**64 - 1), _ptr(positions), _ptr(token),
                           _ptr(kept), _stream(stream)))
    return token, kept


@_on_stream
def gather_rows(head: Head, ids, out: Optional[Head] = None, stream=None):
    """The subset head of `head` (BF16 or FP8_ROW) whose row j is row ids[j] (int32);
    written into `out` when given."""
    _want(ids, torch.int32, "ids")
    n = ids.numel()
    dev = head.weight.device
    if out is None:
        weight = torch.empty((n, head.hidden), dtype=head.weight.dtype, device=dev)
        scale = (torch.empty((n,), dtype=torch.float32, device=dev)
                 if head.format == FP8_ROW else None)
    else:
        weight, scale = out.weight, out.scale
        if weight.shape != (n, head.hidden) or weight.dtype != head.weight.dtype:
            raise ValueError("out: weight must be [len(ids)][H] of the head's dtype")
        _want(weight, weight.dtype, "out.weight")
        if scale is not None:
            _want(scale, torch.float32, "out.scale")
            if scale.numel() != n:
                raise ValueError("out: scale must hold len(ids) floats")
    h = head._c()
    _check(lib().dh_gather_rows(ctypes.byref(h), _ptr(ids), n, _ptr(weight), _ptr(scale),
                                _stream(stream)))
    return Head(head.format, weight, scale)


def rescore_sync_buffer(device="cuda"):
    """A zero-filled sync buffer for rescore(..., sync=) (dh_rescore_sync)."""
    return torch.zeros(RESCORE_SYNC_BYTES, dtype=torch.uint8, device=device)


@_on_stream
def rescore(dense: Head, x, cand_ids, exact=None, draft=None, sync=None, stream=None):
    """(exact fp32 [R][cand_k], draft int32 [R]).  With `sync` (rescore_sync_buffer()), one
    launch: dh_rescore_sync; calls sharing it must be ordered (one stream)."""
    _want(cand_ids, torch.int32, "cand_ids")
    R, ck = cand_ids.shape
    _shaped(x, (R, dense.hidden), BF16_BITS, "x")
    dev = x.device
    exact = torch.empty((R, ck), dtype=torch.float32, device=dev) if exact is None else exact
    draft = torch.empty((R,), dtype=torch.int32, device=dev) if draft is None else draft
    _shaped(exact, (R, ck), torch.float32, "exact")
    _shaped(draft, (R,), torch.int32, "draft")
    h = dense._c()
    if sync is not None:
        _shaped(sync, (RESCORE_SYNC_BYTES,), torch.uint8, "sync")
        _check(lib().dh_rescore_sync(ctypes.byref(h), _ptr(x), R, _ptr(cand_ids), ck,
                                     _ptr(exact), _ptr(draft), _ptr(sync), _stream(stream)))
    else:
        _check(lib().dh_rescore(ctypes.byref(h), _ptr(x), R, _ptr(cand_ids), ck, _ptr(exact),
                                _ptr(draft), _stream(stream)))
    return exact, draft


def _check_outs(o, R, k, vocab):
    _shaped(o["ids"], (R, k), torch.int32, "ids")
    _shaped(o["vals"], (R, k), torch.float32, "vals")
    _shaped(o["draft"], (R,), torch.int32, "draft")
    _shaped(o.get("exact"), (R, k), torch.float32, "exact")
    _shaped(o.get("logits"), (R, vocab), torch.float32, "logits")


@_on_stream
def draft(head: Head, x, k, dense: Optional[Head] = None, ws=None, keep_logits=False,
          out=None, stream=None, idmap=None):
    """The whole projection: dict with ids, vals, draft (+ exact, logits).  With `idmap`
    (int32 [head.vocab]) the head is a subset head and the call is dh_draft_mapped."""
    R = x.shape[0]
    dev = x.device
    o = {} if out is None else out
    o.setdefault("ids", torch.empty((R, k), dtype=torch.int32, device=dev))
    o.setdefault("vals", torch.empty((R, k), dtype=torch.float32, device=dev))
    o.setdefault("draft", torch.empty((R,), dtype=torch.int32, device=dev))
    if dense is not None:
        o.setdefault("exact", torch.empty((R, k), dtype=torch.float32, device=dev))
    if keep_logits:
        o.setdefault("logits", torch.empty((R, head.vocab), dtype=torch.float32, device=dev))
    _shaped(x, (R, head.hidden), BF16_BITS, "x")
    _check_outs(o, R, k, head.vocab)
    ws = workspace(R, head.vocab, k, dev) if ws is None else ws
    h = head._c()
    d = dense._c() if dense is not None else None
    tail = (_ptr(x), R, k, _ptr(o["ids"]), _ptr(o["vals"]), _ptr(o["draft"]),
            _ptr(o.get("exact")), _ptr(o.get("logits")), _ptr(ws), _ws_bytes(ws),
            _stream(stream))
    dref = ctypes.byref(d) if d is not None else None
    if idmap is None:
        _check(lib().dh_draft(ctypes.byref(h), dref, *tail))
    else:
        _want(idmap, torch.int32, "idmap")
        if idmap.numel() != head.vocab:
            raise ValueError(f"idmap: expected {head.vocab} ids, got {idmap.numel()}")
        _check(lib().dh_draft_mapped(ctypes.byref(h), _ptr(idmap), dref, *tail))
    return o


@_on_stream
def draft_noalloc(head: Head, x, k, dense: Optional[Head] = None, keep_logits=False, out=None,
                  stream=None):
    """dh_draft_noalloc: dh_draft on the library's fixed device scratch (no workspace).  The
    library call allocates nothing; pass every output in `out` (ids, vals, draft, and exact
    with `dense`, logits with keep_logits) to make the whole call allocation-free, since
    missing outputs are allocated here.  Calls that overlap on one GPU race."""
    R = x.shape[0]
    dev = x.device
    o = {} if out is None else out
    o.setdefault("ids", torch.empty((R, k), dtype=torch.int32, device=dev))
    o.setdefault("vals", torch.empty((R, k), dtype=torch.float32, device=dev))
    o.setdefault("draft", torch.empty((R,), dtype=torch.int32, device=dev))
    if dense is not None:
        o.setdefault("exact", torch.empty((R, k), dtype=torch.float32, device=dev))
    if keep_logits:
        o.setdefault("logits", torch.empty((R, head.vocab), dtype=torch.float32, device=dev))
    _shaped(x, (R, head.hidden), BF16_BITS, "x")
    _check_outs(o, R, k, head.vocab)
    h = head._c()
    d = dense._c() if dense is not None else None
    _check(lib().dh_draft_noalloc(ctypes.byref(h), ctypes.byref(d) if d is not None else None,
                                  _ptr(x), R, k, _ptr(o["ids"]), _ptr(o["vals"]),
                                  _ptr(o["draft"]), _ptr(o.get("exact")), _ptr(o.get("logits")),
                                  _stream(stream)))
    return o


@_on_stream
def draft_lowrank(down: Head, up: Head, x, k, dense: Optional[Head] = None, ws=None,
                  keep_logits=False, out=None, stream=None):
    """dh_draft_lowrank: t = bf16(x down^T), logits = t up^T, then the draft (dict with ids,
    vals, draft, t (+ exact, logits))."""
    R = x.shape[0]
    dev = x.device
    o = {} if out is None else out
    o.setdefault("ids", torch.empty((R, k), dtype=torch.int32, device=dev))
    o.setdefault("vals", torch.empty((R, k), dtype=torch.float32, device=dev))
    o.setdefault("draft", torch.empty((R,), dtype=torch.int32, device=dev))
    o.setdefault("t", torch.empty((R, down.vocab), dtype=torch.int16, device=dev))
    if dense is not None:
        o.setdefault("exact", torch.empty((R, k), dtype=torch.float32, device=dev))
    if keep_logits:
        o.setdefault("logits", torch.empty((R, up.vocab), dtype=torch.float32, device=dev))
    _shaped(x, (R, down.hidden), BF16_BITS, "x")
    _shaped(o["t"], (R, down.vocab), BF16_BITS, "t")
    _check_outs(o, R, k, up.vocab)
    ws = workspace(R, up.vocab, k, dev) if ws is None else ws
    hd, hu = down._c(), up._c()
    d = dense._c() if dense is not None else None
    _check(lib().dh_draft_lowrank(
        ctypes.byref(hd), ctypes.byref(hu), ctypes.byref(d) if d is not None else None,
        _ptr(x), R, k, _ptr(o["t"]), _ptr(o["ids"]), _ptr(o["vals"]), _ptr(o["draft"]),
        _ptr(o.get("exact")), _ptr(o.get("logits")), _ptr(ws), _ws_bytes(ws), _stream(stream)))
    return o


def draft_mapped(head: Head, idmap, x, k, dense: Optional[Head] = None, **kw):
    """dh_draft_mapped: draft on a subset head whose row j is vocabulary id idmap[j]."""
    return draft(head, x, k, dense=dense, idmap=idmap, **kw)


@_on_stream
def quantize(w, format, stream=None):
    """FP8 head from a bf16 head [V][H]: (codes uint8 [V][H], scale); with format | TILED the
    codes come straight in the tiled layout (a flat uint8 buffer, as tile() makes)."""
    if w.dtype not in (torch.bfloat16, torch.int16):
        raise TypeError("w must be bfloat16 (or its int16 bits)")
    _want(w, w.dtype, "w")
    V, H = w.shape
    base = format & ~TILED
    if format & TILED:
        n = tiled_bytes(format, V, H)
        if n == 0:
            raise DHError(2, "sizes outside the library's limits")
        codes = torch.empty((n,), dtype=torch.uint8, device=w.device)
    else:
        codes = torch.empty((V, H), dtype=torch.uint8, device=w.device)
    if base == FP8_BLOCK32:
        scale = torch.empty(((V + 31) // 32, H // 32), dtype=torch.uint8, device=w.device)
    elif base == FP8_ROW:
        scale = torch.empty((V,), dtype=torch.float32, device=w.device)
    else:
        raise ValueError("format must be FP8_BLOCK32 or FP8_ROW (optionally | TILED)")
    _check(lib().dh_quantize(format, _ptr(w), V, H, _ptr(codes), _ptr(scale), _stream(stream)))
    return codes, scale


STREAM_SINK_WORDS = 8192


@_on_stream
def stream_read(buf, sink=None, stream=None):
    """dh_stream_read: a diagnostic read of a device buffer (uint8, size a multiple of 4096)
    the way the GEMV streams a tiled head; returns the sink (int32 [STREAM_SINK_WORDS]) whose
    words sum, mod 2^32, to the sum of the buffer's 32-bit words."""
    _want(buf, buf.dtype, "buf")
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.empty((STREAM_SINK_WORDS,), dtype=torch.int32, device=buf.device)
    _shaped(sink, (STREAM_SINK_WORDS,), torch.int32, "sink")
    _check(lib().dh_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)))
    return sink


def status_string(status):
    return lib().dh_status_string(status).decode()
