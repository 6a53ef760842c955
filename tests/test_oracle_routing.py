"""Pins of the oracle's router, top-k and tile placement.

* Router GEMV: exact special case (one-hot router rows give back x entries)
  and an independent compensated sum (math.fsum) on small shapes.
* Top-k: an independent selection (K rounds of arg-max, ties to the lower id)
  and the ordering invariants.
* Placement: re-derived by a stable argsort of the row-major expert ids, and
  checked by an invariant checker that is itself shown to catch planted
  mistakes.
"""
import math

import numpy as np
import pytest

from checks import check_placement, check_topk
from moe_decode_layer_amd import synth
from oracle import moe_oracle as O


def test_router_one_hot_rows_give_back_x():
    rng = np.random.default_rng(0)
    T, H, E = 5, 64, 16
    X = O.bf16_round(rng.standard_normal((T, H)))
    pick = rng.choice(H, E, replace=False)
    Wr = np.zeros((E, H), np.float32)
    Wr[np.arange(E), pick] = 1.0
    l = O.router_logits(X, Wr)
    assert np.array_equal(l, X[:, pick])
    idx, _ = O.select_topk(O.sigmoid(l), 3)
    for t in range(T):
        want = sorted(range(E), key=lambda e: -X[t, pick[e]])[:3]
        assert list(idx[t]) == want


def test_router_matches_compensated_sum():
    rng = np.random.default_rng(1)
    T, H, E = 3, 96, 7
    X = O.bf16_round(rng.standard_normal((T, H)))
    Wr = rng.standard_normal((E, H)).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    l = O.router_logits(X, Wr, b)
    for t in range(T):
        for e in range(E):
            ref = math.fsum([X[t, h] * float(Wr[e, h]) for h in range(H)] + [float(b[e])])
            assert abs(l[t, e] - ref) <= 1e-13 * max(1.0, abs(ref))


def _argmax_rounds(scores, K):
    """Independent top-k: K rounds of 'largest remaining score, lowest id on ties'."""
    T, E = scores.shape
    out = np.zeros((T, K), np.int64)
    for t in range(T):
        taken = set()
        for k in range(K):
            best = None
            for e in range(E):
                if e in taken:
                    continue
                if best is None or scores[t, e] > scores[t, best]:
                    best = e
            taken.add(best)
            out[t, k] = best
    return out


@pytest.mark.parametrize("E,K", [(16, 2), (16, 16), (1, 1), (64, 8)])
def test_topk_matches_argmax_rounds(E, K):
    rng = np.random.default_rng(E * 100 + K)
    s = O.sigmoid(rng.standard_normal((20, E)))
    s[3, : E // 2] = 0.5                     # ties resolved to the lower id
    idx, w = O.select_topk(s, K)
    assert np.array_equal(idx, _argmax_rounds(s, K))
    check_topk(s, idx, w, K)
    if K == E:
        assert np.allclose(w, s[np.arange(20)[:, None], idx] / s.sum(axis=1, keepdims=True))


def test_topk_on_logits_equals_topk_on_scores():
    rng = np.random.default_rng(5)
    l = rng.standard_normal((30, 32)) * 3
    i1, _ = O.select_topk(O.sigmoid(l), 4)
    i2, _ = O.select_topk(l, 4)               # sigmoid is monotone
    assert np.array_equal(i1, i2)


def _stable_argsort_ranks(idx, E):
    """Ranks from a stable sort of the row-major flattened expert ids."""
    T, K = idx.shape
    flat = idx.reshape(-1)
    order = np.argsort(flat, kind="stable")
    rank = np.zeros(T * K, np.int64)
    start = 0
    for e in range(E):
        n = int((flat == e).sum())
        rank[order[start:start + n]] = np.arange(n)
        start += n
    return rank.reshape(T, K), np.bincount(flat, minlength=E)


@pytest.mark.parametrize("T,E,K", [(4, 16, 2), (64, 256, 8), (384, 256, 8), (70, 3, 2), (1, 8, 8)])
def test_placement_matches_stable_sort(T, E, K):
    rng = np.random.default_rng(T + E)
    # skewed random choices so some experts need several tiles
    p = 1.0 / np.arange(1, E + 1) ** 1.2
    idx = np.stack([rng.choice(E, K, replace=False, p=p / p.sum()) for _ in range(T)]).astype(np.int32)
    plc = O.place(idx, E)
    rank, count = _stable_argsort_ranks(idx, E)
    assert np.array_equal(plc.rank, rank)
    assert np.array_equal(plc.count, count)
    check_placement(idx, plc.rank, plc.count, E)
    # tiles: each expert's rows in order, 8 at a time
    n_tiles = sum((int(c) + 7) // 8 for c in count)
    assert len(plc.tiles) == n_tiles
    for e, j, rows in plc.tiles:
        assert 1 <= len(rows) <= 8
        for t in rows:
            k = list(idx[t]).index(e)
            assert plc.rank[t, k] // 8 == j


def test_placement_brute_force_tiny():
    idx = np.array([[3, 1], [1, 0], [3, 1], [2, 3]], np.int32)
    plc = O.place(idx, 4)
    assert list(plc.count) == [1, 3, 1, 3]
    assert plc.rank.tolist() == [[0, 0], [1, 0], [1, 2], [0, 2]]
    assert plc.tiles == [(0, 0, (1,)), (1, 0, (0, 1, 2)), (2, 0, (3,)), (3, 0, (0, 2, 3))]


def test_placement_checker_catches_planted_mistakes():
    rng = np.random.default_rng(9)
    idx = np.stack([rng.choice(8, 3, replace=False) for _ in range(40)]).astype(np.int32)
    plc = O.place(idx, 8)
    check_placement(idx, plc.rank, plc.count, 8)
    mutations = []
    r = plc.rank.copy(); r[5, 1] += 1; mutations.append((r, plc.count))          # off by one
    r = plc.rank.copy()
    e = idx[0, 0]
    t2, k2 = next((t, k) for t in range(1, 40) for k in range(3) if idx[t, k] == e)
    r[0, 0], r[t2, k2] = r[t2, k2], r[0, 0]; mutations.append((r, plc.count))    # order broken
    c = plc.count.copy(); c[2] += 1; c[3] -= 1; mutations.append((plc.rank, c))  # counts moved
    r = plc.rank.copy(); r[7, 0] = r[7, 0] + 8; mutations.append((r, plc.count))  # wrong tile
    for r, c in mutations:
        with pytest.raises(AssertionError):
            check_placement(idx, r, c, 8)


@pytest.mark.parametrize("i", range(len(synth.WORKLOADS)))
def test_workload_routing_margins_and_invariants(i):
    wl = synth.WORKLOADS[i]
    Wr = synth.router_weights(wl)
    b = synth.zipf_bias(wl)
    att = O.choose_attempts(wl, lambda a: synth.x_rows(wl, a), Wr, b)
    X = O.bf16_bits_to_f64(synth.x_rows(wl, att))
    s = O.sigmoid(O.router_logits(X, Wr, b))
    assert np.all(O.topk_margins(s, wl.K) >= O.MARGIN)
    idx, w = O.select_topk(s, wl.K)
    check_topk(s, idx, w, wl.K)
    plc = O.place(idx, wl.E)
    check_placement(idx, plc.rank, plc.count, wl.E)
    if wl.zipf_s is not None:
        assert plc.count.max() > 8            # hot experts need several tiles


# --------------------------------------------------------------------------
# The input selection: margins among the top K+1 scores and the redraw loop
# --------------------------------------------------------------------------
@pytest.mark.parametrize("row,accepted", [
    # the gap at the K/K+1 boundary is 5e-4: the top-2 set is ambiguous
    ([0.9, 0.8, 0.7995, 0.1], False),
    # the gap inside the top 2 is 5e-4: the order of the pair is ambiguous
    ([0.9, 0.8995, 0.5, 0.1], False),
    # the only small gap lies past the K+1-th score: irrelevant to the top 2
    ([0.9, 0.8, 0.7, 0.6995], True),
    # the same three rows with the experts in another order (the gaps are
    # taken between scores in rank order, not between neighbouring ids)
    ([0.7995, 0.1, 0.9, 0.8], False),
    ([0.5, 0.8995, 0.1, 0.9], False),
    ([0.6995, 0.7, 0.8, 0.9], True),
])
def test_topk_margins_hand_built_rows(row, accepted):
    s = np.array([row], np.float64)
    m = O.topk_margins(s, 2)
    assert (m[0] >= O.MARGIN) == accepted
    gaps = {(0.9, 0.8, 0.7995, 0.1): 0.0005, (0.9, 0.8995, 0.5, 0.1): 0.0005, (0.9, 0.8, 0.7, 0.6995): 0.1}
    assert m[0] == pytest.approx(gaps[tuple(sorted(row, reverse=True))], abs=1e-12)


def test_topk_margins_when_k_equals_e_uses_the_top_k():
    # K = E: every expert is selected, only the order among them matters
    s = np.array([[0.3, 0.9, 0.6]])
    assert O.topk_margins(s, 3)[0] == pytest.approx(0.3)
    assert O.topk_margins(np.array([[0.5]]), 1)[0] == np.inf


def _stub_workload(T, K):
    return synth.Workload("stub", T=T, H=3, E=3, K=K, S=0, I=32)


def _stub_rows(table):
    """x_rows stand-in: row t of attempt a is table[t][a] (fp64 values, stored
    as bf16 bits).  With the one-hot router below, logits equal x."""
    def rows(att):
        return np.stack([O.bf16_value_to_bits(np.asarray(table[t][min(int(a), len(table[t]) - 1)],
                                                         np.float64))
                         for t, a in enumerate(att)])
    return rows


def test_choose_attempts_redraws_tied_rows_only():
    eye = np.eye(3, dtype=np.float32)         # logits = x
    # row 0: attempt 0 ties experts 0 and 1 at the top, attempt 1 does not;
    # row 1: attempt 0 is already clear; row 2 needs two redraws
    table = [
        [[1.0, 1.0, 0.0], [2.0, 1.0, 0.0]],
        [[0.0, 1.0, 2.0]],
        [[1.0, 0.0, 1.0], [0.5, 0.5, -1.0], [3.0, 0.0, -2.0]],
    ]
    att = O.choose_attempts(_stub_workload(3, 1), _stub_rows(table), eye, None)
    assert att.tolist() == [1, 0, 2]


def test_choose_attempts_fails_loudly_after_max_attempts():
    eye = np.eye(3, dtype=np.float32)
    table = [[[1.0, 1.0, 0.0]]]               # every attempt ties
    with pytest.raises(RuntimeError):
        O.choose_attempts(_stub_workload(1, 1), _stub_rows(table), eye, None, max_attempts=5)


def test_choose_attempts_checks_the_k_plus_1_boundary():
    # K = 2: attempt 0 has a clear top 2 but the 2nd and 3rd scores tie,
    # so the selected set is ambiguous and the row is redrawn
    eye = np.eye(3, dtype=np.float32)
    table = [[[2.0, 1.0, 1.0], [2.0, 1.0, -1.0]]]
    att = O.choose_attempts(_stub_workload(1, 2), _stub_rows(table), eye, None)
    assert att.tolist() == [1]
