"""Comparison rules between the GPU path and the CPU oracle (test code).

Logits: tol_r = 1e-3 * max over the oracle's finite logits of row r of |logit|; every finite
oracle logit must be matched within tol_r, NaN positions must agree, infinities must agree
in sign.

Top-k (k-th boundary gap rule): with L_k the oracle's k-th eligible value and gap_k =
L_k - L_{k+1} (+inf when the row has <= k eligible logits):
 * gap_k > 2 tol_r: the GPU's ids equal the oracle's as a set (pads included); their order
   must agree wherever the oracle's neighbouring values differ by more than 2 tol_r;
 * otherwise membership: every id with L_v > L_k + 2 tol_r is returned, every returned id
   has L_v >= L_k - 2 tol_r, the number of eligible entries is min(k, n_eligible), and the
   GPU list is ordered under its own values.
Pads are (id 0, -inf) in both cases.
"""
import numpy as np


def row_tol(oracle_row, rel=1e-3):
    f = oracle_row[np.isfinite(oracle_row)]
    return rel * (float(np.abs(f).max()) if f.size else 0.0)


def eligible(v):
    v = np.asarray(v)
    return ~np.isnan(v) & (v != -np.inf)


# The largest observed |gpu - oracle| / tol over every checked row of the session (reported by
# conftest.py at the end of the run).
WORST = {"ratio": 0.0, "what": None}


def check_logits(gpu, orc, rel=1e-3, what="logits"):
    """Asserts the logit rule; returns the per-row tolerances."""
    gpu = np.asarray(gpu, np.float32)
    orc = np.asarray(orc, np.float32)
    assert gpu.shape == orc.shape, (gpu.shape, orc.shape)
    tols = []
    for r in range(orc.shape[0]):
        g, o = gpu[r], orc[r]
        tol = row_tol(o, rel)
        tols.append(tol)
        nan_o, nan_g = np.isnan(o), np.isnan(g)
        assert np.array_equal(nan_o, nan_g), f"{what} row {r}: NaN positions differ " \
            f"({np.count_nonzero(nan_o != nan_g)} of {o.size})"
        inf_o = np.isinf(o)
        assert np.array_equal(inf_o, np.isinf(g)), f"{what} row {r}: inf positions differ"
        assert np.array_equal(np.sign(o[inf_o]), np.sign(g[inf_o])), f"{what} row {r}: inf sign"
        fin = np.isfinite(o)
        if fin.any():
            err = np.abs(g[fin].astype(np.float64) - o[fin].astype(np.float64))
            worst = float(err.max())
            assert worst <= tol, f"{what} row {r}: max abs err {worst:.3e} > tol {tol:.3e}"
            if tol > 0 and worst / tol > WORST["ratio"]:
                WORST["ratio"] = worst / tol
                WORST["what"] = f"{what} row {r}: {worst:.3e} of tol {tol:.3e}"
    return np.array(tols)


def _oracle_order(orc_row):
    """Eligible ids of a row sorted by (value desc, id asc)."""
    e = np.nonzero(eligible(orc_row))[0]
    vals = orc_row[e].astype(np.float64)
    order = np.lexsort((e, -vals))
    return e[order]


def check_topk_row(ids, vals, orc_row, k, tol, r=0, what="top-k"):
    """The gap rule for one row.  ids/vals: the GPU's [k] outputs; orc_row: the oracle's
    logits of that row.  Returns 'exact' or 'membership'."""
    ids = np.asarray(ids)
    vals = np.asarray(vals, np.float32)
    order = _oracle_order(orc_row)
    n = order.size
    kk = min(k, n)
    # pads
    assert np.all(ids[kk:] == 0), f"{what} row {r}: pad ids"
    assert np.all(vals[kk:] == -np.inf), f"{what} row {r}: pad values"
    gi = ids[:kk]
    assert np.all(eligible(vals[:kk])), f"{what} row {r}: ineligible value among the first {kk}"
    assert len(set(gi.tolist())) == kk, f"{what} row {r}: repeated ids"
    # own ordering of the GPU list: values non-increasing, ties by id
    gv = vals[:kk].astype(np.float64)
    for j in range(kk - 1):
        assert gv[j] > gv[j + 1] or (gv[j] == gv[j + 1] and gi[j] < gi[j + 1]), \
            f"{what} row {r}: GPU list not ordered at {j}"
    if kk == 0:
        return "exact"
    ov = orc_row.astype(np.float64)
    Lk = ov[order[kk - 1]]
    # equal neighbours (+inf ones included) are 0 apart, not inf - inf
    step = lambda a, b: 0.0 if a == b else a - b
    gap = step(ov[order[kk - 1]], ov[order[kk]]) if n > k else np.inf
    if gap > 2 * tol:
        assert set(gi.tolist()) == set(order[:kk].tolist()), \
            f"{what} row {r}: id set differs from the oracle (gap {gap:.3e} > 2tol {2*tol:.3e})"
        # clusters of oracle values closer than 2 tol may be permuted
        cl = np.zeros(kk, np.int64)
        for j in range(1, kk):
            cl[j] = cl[j - 1] + (step(ov[order[j - 1]], ov[order[j]]) > 2 * tol)
        cluster = {int(v): int(c) for v, c in zip(order[:kk], cl)}
        seq = np.array([cluster[int(v)] for v in gi])
        assert np.array_equal(seq, cl), f"{what} row {r}: order differs across separated values"
        return "exact"
    must = order[ov[order] > Lk + 2 * tol]
    assert set(must.tolist()) <= set(gi.tolist()), f"{what} row {r}: a clear member is missing"
    assert np.all(ov[gi] >= Lk - 2 * tol), f"{what} row {r}: a returned id is clearly out"
    return "membership"


def check_topk(ids, vals, orc_logits, k, tols, what="top-k"):
    kinds = []
    for r in range(orc_logits.shape[0]):
        kinds.append(check_topk_row(ids[r], vals[r], orc_logits[r], k, tols[r], r, what))
    return kinds
