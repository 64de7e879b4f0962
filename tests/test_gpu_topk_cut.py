"""dh_topk's cut path (a cut of each contiguous chunk of a row, then the merge of the cuts) on
the inputs that make a chunk's cut miss keys of the row's top k, so that the merge must read
that chunk back: bit-exact against the oracle's top-k on the same logits."""
import numpy as np
import pytest

import oracle
from few_row_vocab_amd import dh
from gpu_util import dev, host, need_gpu, say

pytestmark = pytest.mark.gpu


def check(logits, k, idmap=None):
    if idmap is None:
        ids, vals, am = dh.topk(dev(logits), k)
        oi, ov = oracle.topk(logits, k)
    else:
        ids, vals, am = dh.topk_mapped(dev(logits), k, dev(idmap))
        oi, ov = oracle.topk_mapped(logits, k, idmap)
    gi, gv = host(ids), host(vals)
    assert np.array_equal(gi, oi)
    assert np.array_equal(gv.view(np.uint32), ov.view(np.uint32))
    assert np.array_equal(host(am), oi[:, 0])


def rows_with(V, R, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((R, V)).astype(np.float32)


@pytest.mark.parametrize("k", [8, 64, 512])
@pytest.mark.parametrize("R", [1, 16])
def test_topk_all_in_one_chunk(R, k):
    """Every one of the k best logits sits in one chunk (a run of ids), more than its cut holds;
    in another row the run straddles two chunks; in a third it is the row's last ids."""
    need_gpu()
    V = 129280
    say(f"topk cut: clustered R={R} k={k}")
    x = rows_with(V, R, seed=R * 10 + k)
    for r in range(R):
        start = [1000, 2 * 2032 - k // 2, V - k][r % 3]   # 2032: a 16-row chunk
        x[r, start:start + k] = 10.0 + np.arange(k, dtype=np.float32) * 1e-3
    check(x, k)


@pytest.mark.parametrize("k", [1, 64, 512])
def test_topk_all_tied(k):
    """All-equal rows (every chunk's cut is empty: the whole row is read back), one with a
    single larger value, one of zeros of both signs."""
    need_gpu()
    V = 70001
    x = np.full((3, V), 0.5, np.float32)
    x[1, 12345] = 0.75
    x[2] = 0.0
    x[2, ::2] = -0.0
    check(x, k)


@pytest.mark.parametrize("k", [64, 512])
def test_topk_crowded_boundary(k):
    """Many logits equal to the k-th largest, spread over every chunk: ties go to the lower
    ids, across chunk boundaries."""
    need_gpu()
    V = 129280
    x = rows_with(V, 4, seed=k)
    x[:, ::97] = 3.0                       # ~1333 equal values above the rest
    x[1, ::2] = 3.0                        # half the row equal
    x[2, 5000:5000 + 4 * k] = 4.0          # a run of equal maxima in one chunk
    check(x, k)


def test_topk_cut_mapped_and_largest_vocab():
    """The id map through the cut path; the largest vocabulary (V = 262,144, 16-entry
    chunks of 1024) with 16 rows."""
    need_gpu()
    V = 49152
    rng = np.random.default_rng(5)
    idmap = np.sort(rng.choice(131072, V, replace=False)).astype(np.int32)
    x = rows_with(V, 5, seed=6)
    x[0, 100:164] = 9.0 + np.arange(64, dtype=np.float32)
    check(x, 64, idmap)
    x = rows_with(dh.MAX_VOCAB, 16, seed=7)
    x[3, -300:] = 7.0
    check(x, 512)
    check(x, 1)


def _shapes():
    """Seeded (rows, V, k) cases across the cut's chunk rule (1024 / rows chunks, between 64
    and 256, fewer when the row has fewer 16-entry tiles): ragged V, tiny V, V just past a
    chunk boundary, every row count from 1 to 32."""
    rng = np.random.default_rng(2024)
    out = [(1, 17, 17), (2, 1023, 64), (5, 4111, 512), (8, 16385, 100), (17, 9000, 33),
           (32, 2049, 64), (3, 262144, 1), (12, 131071, 255)]
    for _ in range(8):
        R = int(rng.integers(1, 33))
        V = int(rng.integers(20, 200000))
        k = int(min(V, rng.choice([1, 7, 64, 65, 200, 512])))
        out.append((R, V, k))
    return out


@pytest.mark.parametrize("R,V,k", _shapes())
def test_topk_cut_random_shapes(R, V, k):
    """Planted rows (NaN, -inf, ties, +-0, subnormals, ascending, descending, few eligible,
    winners straddling chunks or in one chunk) at seeded shapes: bit-exact."""
    need_gpu()
    from test_gpu_core import _planted
    say(f"topk cut: R={R} V={V} k={k}")
    check(_planted(R, V, seed=R * 7919 + V + k), k)
