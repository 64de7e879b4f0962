"""CPU oracle of the few-row draft-head vocabulary projection -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg may
import this package.  The product library (``few_row_vocab_amd``) never does, and it shares
no code with it.  This module marshals numpy arrays into ``liboracle.so`` (oracle.c, plain C
in double precision); every definition lives, with its citation, in oracle.c.

Parity pins: see tests/test_oracle_*.py.  Functions without an independent pin: the readings
for rescore pads and out-of-range candidate ids (``rescore``), which are "parity unpinned"
beyond their own definitions.
"""
import ctypes
import os

import numpy as np

from . import build as _build

FMT_BF16 = 0
FMT_FP8_BLOCK32 = 1
FMT_FP8_ROW = 2

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        c = ctypes
        L.orc_bf16_value.restype = c.c_double
        L.orc_bf16_value.argtypes = [c.c_uint16]
        L.orc_e4m3_value.restype = c.c_double
        L.orc_e4m3_value.argtypes = [c.c_uint8]
        L.orc_e8m0_value.restype = c.c_double
        L.orc_e8m0_value.argtypes = [c.c_uint8]
        L.orc_e4m3_encode.restype = c.c_uint8
        L.orc_e4m3_encode.argtypes = [c.c_float]
        L.orc_beats.restype = c.c_int
        L.orc_beats.argtypes = [c.c_float, c.c_int64, c.c_float, c.c_int64]
        L.orc_gemv.restype = None
        L.orc_gemv.argtypes = [c.c_int, c.c_void_p, c.c_void_p, c.c_int64, c.c_int64,
                               c.c_void_p, c.c_int, c.c_void_p, c.c_int64, c.c_void_p]
        L.orc_topk.restype = c.c_int
        L.orc_topk.argtypes = [c.c_void_p, c.c_int, c.c_int64, c.c_int, c.c_void_p,
                               c.c_void_p]
        L.orc_topk_mapped.restype = c.c_int
        L.orc_topk_mapped.argtypes = [c.c_void_p, c.c_int, c.c_int64, c.c_int, c.c_void_p,
                                      c.c_void_p, c.c_void_p]
        L.orc_topk_softmax.restype = c.c_int
        L.orc_topk_softmax.argtypes = [c.c_void_p, c.c_int, c.c_int64, c.c_int, c.c_void_p,
                                       c.c_void_p, c.c_void_p, c.c_void_p]
        L.orc_philox4x64.restype = None
        L.orc_philox4x64.argtypes = [c.c_void_p, c.c_void_p, c.c_void_p]
        L.orc_keyed_uniform.restype = c.c_double
        L.orc_keyed_uniform.argtypes = [c.c_uint64, c.c_int64, c.c_int32]
        L.orc_sample.restype = None
        L.orc_sample.argtypes = [c.c_void_p, c.c_void_p, c.c_int, c.c_int, c.c_double,
                                 c.c_double, c.c_double, c.c_uint64, c.c_void_p, c.c_void_p,
                                 c.c_void_p, c.c_void_p]
        L.orc_subset_rows.restype = None
        L.orc_subset_rows.argtypes = [c.c_void_p, c.c_void_p, c.c_int64, c.c_int64, c.c_int,
                                      c.c_void_p, c.c_int64, c.c_void_p, c.c_void_p]
        L.orc_bf16_encode.restype = c.c_uint16
        L.orc_bf16_encode.argtypes = [c.c_double]
        L.orc_linear.restype = None
        L.orc_linear.argtypes = [c.c_int, c.c_void_p, c.c_void_p, c.c_int64, c.c_int64,
                                 c.c_void_p, c.c_int, c.c_int, c.c_void_p, c.c_void_p]
        L.orc_rescore.restype = None
        L.orc_rescore.argtypes = [c.c_void_p, c.c_int64, c.c_int64, c.c_void_p, c.c_int,
                                  c.c_void_p, c.c_void_p, c.c_int, c.c_void_p, c.c_void_p]
        L.orc_quant_row.restype = None
        L.orc_quant_row.argtypes = [c.c_void_p, c.c_int64, c.c_int64, c.c_void_p,
                                    c.c_void_p]
        L.orc_quant_block32.restype = None
        L.orc_quant_block32.argtypes = [c.c_void_p, c.c_int64, c.c_int64, c.c_void_p,
                                        c.c_void_p]
        L.orc_threads.restype = c.c_int
        L.orc_threads.argtypes = [c.c_int]
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def bf16_value(b):
    return lib().orc_bf16_value(int(b))


def e4m3_value(c):
    return lib().orc_e4m3_value(int(c))


def e8m0_value(b):
    return lib().orc_e8m0_value(int(b))


def e4m3_encode(f):
    return lib().orc_e4m3_encode(float(np.float32(f)))


def beats(lu, u, lv, v):
    return bool(lib().orc_beats(float(np.float32(lu)), int(u), float(np.float32(lv)), int(v)))


def gemv(fmt, w, scale, x, vids=None):
    """O5.  w: bf16 bits uint16 [V][H] or E4M3 codes uint8 [V][H]; scale: None, uint8
    [ceil(V/32)][H/32] or float32 [V]; x: bf16 bits uint16 [R][H].  Returns float32
    [R][V] (or [R][len(vids)])."""
    w = np.ascontiguousarray(w)
    V, H = w.shape
    x = _c(x, np.uint16)
    R = x.shape[0]
    if x.shape[1] != H:
        raise ValueError("x width != head width")
    if fmt == FMT_BF16:
        w = _c(w, np.uint16)
        scale = None
    elif fmt == FMT_FP8_BLOCK32:
        w = _c(w, np.uint8)
        scale = _c(scale, np.uint8)
        if scale.shape != ((V + 31) // 32, H // 32):
            raise ValueError("block scale shape")
    elif fmt == FMT_FP8_ROW:
        w = _c(w, np.uint8)
        scale = _c(scale, np.float32)
        if scale.shape != (V,):
            raise ValueError("row scale shape")
    else:
        raise ValueError("format")
    if vids is not None:
        vids = _c(np.asarray(vids, dtype=np.int64), np.int64)
        if vids.size and (vids.min() < 0 or vids.max() >= V):
            raise ValueError("vids out of range")
        nv = vids.size
    else:
        nv = V
    out = np.empty((R, nv), np.float32)
    lib().orc_gemv(fmt, _p(w), _p(scale), V, H, _p(x), R, _p(vids), nv, _p(out))
    return out


def bf16_encode(d):
    """O14a: bf16 bits of a real number (round to nearest even, one rounding)."""
    return int(lib().orc_bf16_encode(float(d)))


MODE_F32, MODE_BF16, MODE_ADD_BF16 = 0, 1, 2


def linear(fmt, w, scale, x, mode, residual=None):
    """O14.  w [N][K] in any storage format (as gemv), x bf16 bits [R][K]; mode 0 -> float32
    [R][N], mode 1 -> bf16 bits [R][N], mode 2 -> bf16 bits of residual + the sum."""
    w = np.ascontiguousarray(w)
    N, K = w.shape
    x = _c(x, np.uint16)
    R = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("x width != weight width")
    if fmt == FMT_BF16:
        w, scale = _c(w, np.uint16), None
    elif fmt == FMT_FP8_BLOCK32:
        w, scale = _c(w, np.uint8), _c(scale, np.uint8)
    elif fmt == FMT_FP8_ROW:
        w, scale = _c(w, np.uint8), _c(scale, np.float32)
    else:
        raise ValueError("format")
    if mode == MODE_ADD_BF16:
        residual = _c(residual, np.uint16)
        if residual.shape != (R, N):
            raise ValueError("residual shape")
    else:
        residual = None
    out = np.empty((R, N), np.float32 if mode == MODE_F32 else np.uint16)
    lib().orc_linear(fmt, _p(w), _p(scale), N, K, _p(x), R, mode, _p(residual), _p(out))
    return out


def topk(logits, k):
    """O8/O9.  logits float32 [R][V] -> (ids int32 [R][k], vals float32 [R][k])."""
    logits = _c(logits, np.float32)
    R, V = logits.shape
    ids = np.empty((R, k), np.int32)
    vals = np.empty((R, k), np.float32)
    if lib().orc_topk(_p(logits), R, V, k, _p(ids), _p(vals)) != 0:
        raise MemoryError("oracle top-k")
    return ids, vals


def topk_softmax(logits, k):
    """O8 + O16: (ids int32 [R][k], vals float32 [R][k], probs float32 [R][k], lse float32
    [R]); probs[:, 0] is the top-1's confidence."""
    logits = _c(logits, np.float32)
    R, V = logits.shape
    ids = np.empty((R, k), np.int32)
    vals = np.empty((R, k), np.float32)
    probs = np.empty((R, k), np.float32)
    lse = np.empty((R,), np.float32)
    if lib().orc_topk_softmax(_p(logits), R, V, k, _p(ids), _p(vals), _p(probs), _p(lse)) != 0:
        raise MemoryError("oracle top-k")
    return ids, vals, probs, lse


def philox4x64(ctr, key):
    """Philox4x64-10 of counter (4 x uint64) and key (2 x uint64): 4 x uint64."""
    c = np.ascontiguousarray(ctr, np.uint64)
    kk = np.ascontiguousarray(key, np.uint64)
    out = np.empty(4, np.uint64)
    lib().orc_philox4x64(_p(c), _p(kk), _p(out))
    return out


def keyed_uniform(seed, position, token):
    return float(lib().orc_keyed_uniform(int(seed), int(position), int(token)))


def sample(ids, vals, T, top_p, min_p, seed, pos):
    """O17: the keyed pick over top-k lists (ids int32 [R][k], vals float32 [R][k]); pos int64
    [R].  -> (token int32 [R], kept int32 [R], score float64 [R][k])."""
    ids = _c(ids, np.int32)
    vals = _c(vals, np.float32)
    R, k = ids.shape
    pos = _c(np.asarray(pos, np.int64), np.int64)
    token = np.empty(R, np.int32)
    kept = np.empty(R, np.int32)
    score = np.empty((R, k), np.float64)
    lib().orc_sample(_p(ids), _p(vals), R, k, float(T), float(top_p), float(min_p),
                     int(seed), _p(pos), _p(token), _p(kept), _p(score))
    return token, kept, score


def topk_mapped(logits, k, idmap):
    """O13.  Top-k of a subset head's logits [R][n] whose column j is token idmap[j]: ids are
    token ids, ties go to the lower token id.  -> (ids int32 [R][k], vals float32 [R][k])."""
    logits = _c(logits, np.float32)
    R, V = logits.shape
    idmap = _c(idmap, np.int32)
    if idmap.shape != (V,):
        raise ValueError("idmap length != logits width")
    ids = np.empty((R, k), np.int32)
    vals = np.empty((R, k), np.float32)
    if lib().orc_topk_mapped(_p(logits), R, V, k, _p(idmap), _p(ids), _p(vals)) != 0:
        raise MemoryError("oracle top-k")
    return ids, vals


def subset_rows(fmt, w, scale, ids):
    """O12.  The subset head of (w, scale) for token ids (int32 [n]): (w' [n][H], scale'
    float32 [n] or None).  Per-row FP8 or bf16; ids outside [0, V) give zero rows."""
    if fmt == FMT_BF16:
        w = _c(w, np.uint16)
        es, scale = 2, None
    elif fmt == FMT_FP8_ROW:
        w = _c(w, np.uint8)
        es = 1
        scale = _c(scale, np.float32)
    else:
        raise ValueError("subset rows: bf16 or per-row FP8 heads only")
    V, H = w.shape
    ids = _c(ids, np.int32)
    n = ids.size
    out = np.empty((n, H), w.dtype)
    out_s = np.empty((n,), np.float32) if scale is not None else None
    lib().orc_subset_rows(_p(w), _p(scale), V, H, es, _p(ids), n, _p(out), _p(out_s))
    return out, out_s


def draft_lowrank(down, up, x, k, dense_w=None, t=None):
    """O15: O11 with a low-rank stage 1 ([TFE] two_stage commit note: the candidates come
    from low-rank logits).  down = (fmt, w [rank][H], scale), up = (fmt, w [V][rank], scale):
    t = O14 mode 1 of x through down (bf16 bits [R][rank]); logits = O5 of t through up;
    then O8 and, with dense_w, O10 from x.  `t` given: the conditional form, which takes
    that t (the GPU's) instead of its own.  Returns dict with t, logits, ids, vals, draft
    (+ exact)."""
    if t is None:
        t = linear(down[0], down[1], down[2], x, MODE_BF16)
    logits = gemv(up[0], up[1], up[2], t)
    ids, vals = topk(logits, k)
    out = {"t": t, "logits": logits, "ids": ids, "vals": vals}
    if dense_w is None:
        out["draft"] = ids[:, 0].copy()
    else:
        exact, d = rescore(dense_w, x, ids, vals > -np.inf)
        out["exact"] = exact
        out["draft"] = d
    return out


def draft_mapped(fmt, w, scale, idmap, x, k, dense_w=None):
    """O11 on a subset head (O12) whose row j is token idmap[j], with O13's top-k; the
    two-stage dense head spans the whole vocabulary."""
    logits = gemv(fmt, w, scale, x)
    ids, vals = topk_mapped(logits, k, idmap)
    out = {"logits": logits, "ids": ids, "vals": vals}
    if dense_w is None:
        out["draft"] = ids[:, 0].copy()
    else:
        use = vals > -np.inf
        exact, d = rescore(dense_w, x, ids, use)
        out["exact"] = exact
        out["draft"] = d
    return out


def argmax(logits):
    return topk(logits, 1)[0][:, 0].copy()


def rescore(dense_w, x, cand, use=None):
    """O10.  dense_w bf16 bits [V][H]; x [R][H]; cand int32 [R][ck]; use uint8/bool [R][ck]
    or None.  Returns (exact float32 [R][ck], draft int32 [R])."""
    dense_w = _c(dense_w, np.uint16)
    V, H = dense_w.shape
    x = _c(x, np.uint16)
    cand = _c(cand, np.int32)
    R, ck = cand.shape
    if use is not None:
        use = _c(np.asarray(use).astype(np.uint8), np.uint8)
    exact = np.empty((R, ck), np.float32)
    draft = np.empty((R,), np.int32)
    lib().orc_rescore(_p(dense_w), V, H, _p(x), R, _p(cand), _p(use), ck, _p(exact),
                      _p(draft))
    return exact, draft


def draft(fmt, w, scale, x, k, dense_w=None):
    """O11.  One stage: top-k of the head's logits and argmax.  Two stage (dense_w given):
    top cand_k = k by the head's logits, then the rescore of the eligible candidates (pads
    are not candidates).  Returns dict with logits, ids, vals, draft (+ exact)."""
    logits = gemv(fmt, w, scale, x)
    ids, vals = topk(logits, k)
    out = {"logits": logits, "ids": ids, "vals": vals}
    if dense_w is None:
        out["draft"] = ids[:, 0].copy()
    else:
        use = vals > -np.inf  # pads of the stage-1 list carry -inf
        exact, d = rescore(dense_w, x, ids, use)
        out["exact"] = exact
        out["draft"] = d
    return out


def quant_row(w_bf16):
    """Q1 -> (codes uint8 [V][H], scale float32 [V])."""
    w = _c(w_bf16, np.uint16)
    V, H = w.shape
    codes = np.empty((V, H), np.uint8)
    scale = np.empty((V,), np.float32)
    lib().orc_quant_row(_p(w), V, H, _p(codes), _p(scale))
    return codes, scale


def quant_block32(w_bf16):
    """Q2 -> (codes uint8 [V][H], scales uint8 [ceil(V/32)][H/32])."""
    w = _c(w_bf16, np.uint16)
    V, H = w.shape
    if H % 32:
        raise ValueError("H must be a multiple of 32")
    codes = np.empty((V, H), np.uint8)
    scales = np.empty(((V + 31) // 32, H // 32), np.uint8)
    lib().orc_quant_block32(_p(w), V, H, _p(codes), _p(scales))
    return codes, scales


def threads(n=0):
    """Threads the oracle's loops use; n > 0 sets that number first."""
    return lib().orc_threads(n)
