"""GPU parity at the library's maximum sizes, through the C ABI.

 * top-k at the largest vocabulary (262,144), the most rows (32) and the largest k (512), on
   planted rows of every kind: bit-exact with the oracle;
 * the GEMV at its largest vocabulary (2^25 rows, H = 32) with 32 rows: a structured bf16 head
   whose values are small multiples of 1/8, so every logit is exact in fp32 and the sampled
   rows must equal the oracle's bit for bit (the oracle computes 4,096 sampled rows);
 * the rescore with the most rows and candidates (32 x 512) against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from few_row_vocab_amd import dh
from gpu_util import dev, dev_u16, host, need_gpu, say
from parity import check_logits
from test_gpu_core import _planted

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def test_topk_max_sizes():
    need_gpu()
    V, R, k = dh.MAX_VOCAB, dh.MAX_ROWS, dh.MAX_K
    say(f"topk V={V} R={R} k={k}")
    logits = _planted(R, V, seed=2024)
    ids, vals, am = dh.topk(dev(logits), k)
    oi, ov = oracle.topk(logits, k)
    assert np.array_equal(host(ids), oi)
    assert np.array_equal(host(vals).view(np.uint32), ov.view(np.uint32))
    assert np.array_equal(host(am), oi[:, 0])


def _structured_head_bits(V, H, seed):
    """bf16 bits of w[v][h] = (((v * a + h * b) mod 17) - 8) / 8: a row depends on v mod 17
    only, so the 17 distinct rows are tiled (a row offset error of anything but a multiple of
    17 changes the logits)."""
    rng = np.random.default_rng(seed)
    a, b = int(rng.integers(3, 97)), int(rng.integers(3, 97))
    table = np.array([np.float32((i - 8) / 8).view(np.uint32) >> 16 for i in range(17)],
                     np.uint16)
    base = table[(np.arange(17)[:, None] * a + np.arange(H)[None, :] * b) % 17]
    return np.tile(base, (-(-V // 17), 1))[:V]


def test_gemv_max_vocab_and_rows():
    need_gpu()
    V, H, R = 1 << 25, 32, dh.MAX_ROWS
    say(f"gemv V={V} H={H} R={R}")
    w = _structured_head_bits(V, H, seed=5)
    rng = np.random.default_rng(6)
    xs = (rng.integers(-4, 5, size=(R, H)) / 4).astype(np.float32)
    x = (xs.view(np.uint32) >> 16).astype(np.uint16)
    head = dh.Head(dh.BF16, dev_u16(w))
    lg = dh.gemv(head, dev_u16(x))
    torch.cuda.synchronize()
    vids = np.sort(rng.choice(V, 4096, replace=False))
    vids[-1] = V - 1                                          # the last row of the last tile
    want = oracle.gemv(oracle.FMT_BF16, w, None, x, vids=vids)
    got = host(lg[:, torch.from_numpy(vids).cuda()])
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_rescore_max_sizes():
    need_gpu()
    V, H, R, ck = 50000, 1024, dh.MAX_ROWS, dh.MAX_K
    w = synth.random_head(V, H, seed=8, std=0.02)
    x = synth.random_acts(R, H, seed=9)
    rng = np.random.default_rng(10)
    cand = rng.integers(0, V, size=(R, ck)).astype(np.int32)
    exact, draft = dh.rescore(dh.Head(dh.BF16, dev_u16(w)), dev_u16(x), dev(cand))
    torch.cuda.synchronize()
    oe, od = oracle.rescore(w, x, cand)
    check_logits(host(exact), oe, what="exact")
    ge = host(exact)
    for r in range(R):
        # the GPU's draft is the best of its own exact logits (ties to the lower id)
        best = np.max(ge[r])
        assert host(draft)[r] == np.min(cand[r][ge[r] == best])
