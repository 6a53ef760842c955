"""Invariant checks of routing and tile placement, plus the output error metrics.

Used on the oracle's results (CPU tests) and on the GPU's debug outputs
(GPU tests).  Written independently of both.
"""
import numpy as np

TILE = 8


def check_topk(scores, idx, w, K, w_tol=1e-12):
    """K distinct experts per row, score-descending, every selected score >=
    every unselected one, weights = selected scores / their sum."""
    T, E = scores.shape
    assert idx.shape == (T, K) and w.shape == (T, K)
    for t in range(T):
        sel = [int(e) for e in idx[t]]
        assert len(set(sel)) == K, f"row {t}: repeated expert"
        assert all(0 <= e < E for e in sel)
        s = scores[t, sel]
        assert np.all(np.diff(s) <= 0), f"row {t}: not score-descending"
        rest = np.delete(scores[t], sel)
        if rest.size:
            assert s.min() >= rest.max(), f"row {t}: an unselected expert scores higher"
        assert abs(w[t].sum() - 1.0) <= w_tol * 10 + 1e-15
        assert np.allclose(w[t], s / s.sum(), rtol=0, atol=w_tol)


def check_placement(idx, rank, count, E):
    """Every (row, k) pair placed exactly once; per expert the ranks are
    0..count-1 in increasing row order (token order preserved); tiles hold at
    most 8 rows and all but an expert's last tile are full; counts sum to T*K."""
    T, K = idx.shape
    assert rank.shape == (T, K) and count.shape == (E,)
    assert int(count.sum()) == T * K
    seen = {}
    for t in range(T):
        for k in range(K):
            e = int(idx[t, k])
            r = int(rank[t, k])
            assert 0 <= r < count[e], f"pair ({t},{k}): rank {r} outside [0,{count[e]})"
            assert (e, r) not in seen, f"pair ({t},{k}) shares slot with {seen[(e, r)]}"
            seen[(e, r)] = (t, k)
    for e in range(E):
        rows = [seen[(e, r)][0] for r in range(int(count[e]))]
        assert rows == sorted(rows) and len(set(rows)) == len(rows), f"expert {e}: order"
        n_tiles = (int(count[e]) + TILE - 1) // TILE
        for j in range(n_tiles):
            filled = min(TILE, int(count[e]) - TILE * j)
            assert 1 <= filled <= TILE
            if j < n_tiles - 1:
                assert filled == TILE


def output_errors(got, want):
    """max|d| / max|o| and sum|d| / sum|o| over all elements, in fp64."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    d = np.abs(got - want)
    return float(d.max() / np.abs(want).max()), float(d.sum() / np.abs(want).sum())


# Output tolerances of the layer (max-relative, mean-relative).
MAX_REL = 1e-2
MEAN_REL = 2e-3
