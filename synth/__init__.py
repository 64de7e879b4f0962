"""Seeded synthetic inputs for the few-row draft-head vocabulary projection.

This module is the only code that both the CPU oracle's callers and the GPU library's callers
use.  It draws random numbers and lays them out; it holds none of the method's arithmetic (no
dot products, no quantization, no ordering).  FP8 heads are made from these bf16 heads by each
side's own quantizer.

Stand-ins: the pages measure trained draft heads (DeepSeek-V4.1's drafter vocabulary head and
a TFE head) that are not available; these generators give heads of the same shapes with
Gaussian entries, which is what the workload descriptions below ask for.

Random stream: numpy PCG64 seeded with ``[seed, stream, block]`` where ``block`` indexes
2**20-element blocks of the flattened array, so any row range can be generated on its own
and blocks can be drawn in parallel.  float32 normals are scaled in float32 and rounded to
bf16 (round to nearest even) by torch's dtype conversion.
"""
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

BLOCK = 1 << 20

STREAM_WEIGHTS = 0
STREAM_ACTS = 1
STREAM_PLANT = 2
STREAM_IDS = 3

# Workloads (shapes from the workload descriptions; seeds are this module's choice).
CONFIGS = {
    "tiny_bf16": dict(H=256, V=4096, rows=[1], fmt="bf16", w_std=None, x="normal_rsqrt_h",
                      ks=[1, 8], seed=101),
    "fp8_block_1row": dict(H=5120, V=129280, rows=[1], fmt="fp8_block32", w_std=0.02,
                           x="normal", ks=[1, 64], seed=202),
    "row_sweep": dict(H=5120, V=129280, rows=[1, 5, 10, 15, 16], fmt="bf16+fp8_block32",
                      w_std=0.02, x="normal", ks=[1, 64], seed=303),
    "two_stage": dict(H=5120, V=129280, rows=[16], fmt="fp8_row+bf16_dense", w_std=0.02,
                      x="normal", ks=[512], seed=404),
    "edge": dict(H=7168, V=163840, rows=[16], fmt="fp8_block32", w_std=0.02, x="edge_grid",
                 ks=[1, 22, 31, 32, 33, 512], seed=505),
    # a low-rank stage 1 (rank 512, bf16 factors) with the dense bf16 head for the rescore
    "lowrank": dict(H=5120, V=129280, rank=512, rows=[16], fmt="bf16", w_std=0.02,
                    x="normal", ks=[512], seed=707),
    # a draft-vocabulary subset: 49,152 of a 131,072-token head of width 4,096, FP8 rows
    "subset_head": dict(H=4096, V=131072, n_draft=49152, rows=[1, 16, 32], fmt="fp8_row",
                        w_std=0.02, x="normal", ks=[1, 64, 512], seed=606),
}

# Edge workload planting (rows of the 16-row activation matrix).
EDGE_ZERO_ROW = 10
EDGE_NAN_ROW = 11
EDGE_PINF_ROW = 12
EDGE_NINF_ROW = 13
EDGE_HOT_ROW = 14
EDGE_HOT_BLOCK = 1234          # 32-row block of identical head rows: rows 39488..39519
GRID = np.array([-2, -1, 0, 1, 2], np.float32) / 8


def _threads():
    return max(1, min(16, os.cpu_count() or 1))


def to_bf16_bits(f32):
    """float32 array -> bf16 bit patterns (uint16), round to nearest even (torch)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b):
    """bf16 bit patterns -> float32 values (exact widening)."""
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_f32(n_total, seed, stream, start=0, stop=None, std=1.0):
    """Elements [start, stop) of a seeded stream of n_total N(0, std^2) float32 values."""
    stop = n_total if stop is None else stop
    out = np.empty(stop - start, np.float32)
    b0, b1 = start // BLOCK, (stop + BLOCK - 1) // BLOCK

    def fill(b):
        lo, hi = b * BLOCK, min((b + 1) * BLOCK, n_total)
        z = np.random.default_rng([seed, stream, b]).standard_normal(hi - lo, np.float32)
        if std != 1.0:
            z *= np.float32(std)
        s, e = max(lo, start), min(hi, stop)
        out[s - start:e - start] = z[s - lo:e - lo]

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(b0, b1)))
    return out


def normal_bf16(shape, seed, stream, std=1.0, row_start=0, row_stop=None):
    """bf16 bits of N(0, std^2) entries of a [V][H] matrix; optionally only rows
    [row_start, row_stop)."""
    V, H = shape
    row_stop = V if row_stop is None else row_stop
    f = normal_f32(V * H, seed, stream, row_start * H, row_stop * H, std)
    return to_bf16_bits(f).reshape(row_stop - row_start, H)


def head_bf16(name, row_start=0, row_stop=None):
    """The bf16 head of a workload (bit patterns, [V][H] or a row range of it)."""
    c = CONFIGS[name]
    V, H = c["V"], c["H"]
    std = c["w_std"] if c["w_std"] is not None else 1.0 / np.sqrt(np.float32(H))
    w = normal_bf16((V, H), c["seed"], STREAM_WEIGHTS, std, row_start, row_stop)
    if name == "edge":
        _plant_hot_block(w, c, row_start)
    return w


def _plant_hot_block(w, c, row_start):
    """Edge workload: the 32 rows of one 32-row block are copies of the block's first row,
    so they share codes and scales and tie exactly in every logit row."""
    H = c["H"]
    src = normal_bf16((c["V"], H), c["seed"], STREAM_WEIGHTS, c["w_std"],
                      EDGE_HOT_BLOCK * 32, EDGE_HOT_BLOCK * 32 + 1)[0]
    for v in range(EDGE_HOT_BLOCK * 32, EDGE_HOT_BLOCK * 32 + 32):
        if row_start <= v < row_start + w.shape[0]:
            w[v - row_start] = src


def activations(name, rows):
    """bf16 bits [rows][H] of a workload's activation rows."""
    c = CONFIGS[name]
    H = c["H"]
    if c["x"] == "normal_rsqrt_h":
        f = normal_f32(rows * H, c["seed"], STREAM_ACTS, std=1.0 / np.sqrt(np.float32(H)))
        return to_bf16_bits(f).reshape(rows, H)
    if c["x"] == "normal":
        return to_bf16_bits(normal_f32(rows * H, c["seed"], STREAM_ACTS)).reshape(rows, H)
    if c["x"] == "edge_grid":
        return edge_activations(c, rows)
    raise ValueError(c["x"])


def edge_activations(c, rows):
    """Rows 0-9 and 15: uniform on {-2,-1,0,1,2}/8.  Row 10: zeros.  Row 11: grid with one
    NaN.  Row 12: grid with one +inf.  Row 13: grid with one -inf.  Row 14: +-1/4 with the
    signs of the hot block's row, so the 32 tied rows lead that logit row."""
    H = c["H"]
    rng = np.random.default_rng([c["seed"], STREAM_PLANT])
    x = GRID[rng.integers(0, 5, size=(16, H))].astype(np.float32)
    x[EDGE_ZERO_ROW] = 0.0
    x[EDGE_NAN_ROW, rng.integers(0, H)] = np.nan
    x[EDGE_PINF_ROW, rng.integers(0, H)] = np.inf
    x[EDGE_NINF_ROW, rng.integers(0, H)] = -np.inf
    hot = bf16_bits_to_f32(head_bf16("edge", EDGE_HOT_BLOCK * 32, EDGE_HOT_BLOCK * 32 + 1)[0])
    x[EDGE_HOT_ROW] = np.where(hot >= 0, np.float32(0.25), np.float32(-0.25))
    return to_bf16_bits(x[:rows]).reshape(rows, H)


def random_head(V, H, seed, std=1.0):
    """A small seeded bf16 head for tests of arbitrary shape."""
    return normal_bf16((V, H), seed, STREAM_WEIGHTS, std)


def random_acts(R, H, seed, std=1.0):
    return to_bf16_bits(normal_f32(R * H, seed, STREAM_ACTS, std=std)).reshape(R, H)


def lowrank_factors(name):
    """(down [rank][H], up [V][rank]) bf16 bits of a low-rank workload: down ~ N(0, 1/H), so
    the rank-r activations of N(0, 1) rows are about N(0, 1), and up ~ N(0, w_std^2)."""
    c = CONFIGS[name]
    H, V, rk = c["H"], c["V"], c["rank"]
    down = normal_bf16((rk, H), c["seed"] + 1, STREAM_WEIGHTS, 1.0 / np.sqrt(np.float32(H)))
    up = normal_bf16((V, rk), c["seed"] + 2, STREAM_WEIGHTS, c["w_std"])
    return down, up


def token_ids(V, n, seed):
    """n distinct token ids of [0, V), drawn uniformly and sorted (int32): the stand-in for a
    draft vocabulary's id list."""
    rng = np.random.default_rng([seed, STREAM_IDS, V, n])
    return np.sort(rng.choice(V, size=n, replace=False)).astype(np.int32)


def draft_ids(name):
    """The draft vocabulary's token ids of a subset workload."""
    c = CONFIGS[name]
    return token_ids(c["V"], c["n_draft"], c["seed"])


def logit_rows(R, V, seed, kind):
    """Planted float32 logit rows for top-k tests (see tests for the list of kinds)."""
    rng = np.random.default_rng([seed, STREAM_PLANT, R, V])
    if kind == "normal":
        return rng.standard_normal((R, V), np.float32)
    if kind == "coarse":      # many exact ties
        return rng.integers(-4, 5, size=(R, V)).astype(np.float32) / 4
    raise ValueError(kind)
