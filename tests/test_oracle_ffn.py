"""Pins of the oracle's expert FFN and weighted combine.

* Dense brute force: every expert evaluated for every row, then masked by
  the top-k weights (zero for unselected experts), written with torch ops
  and torch's own FP8 decoder -- the sparse oracle must agree to fp64
  rounding.
* Special cases: one expert with K = 1 is a plain SwiGLU MLP; K = E is a
  dense mixture weighted by the normalised scores.
* A hand-built case with a closed form (gate and up rows differ, so a
  swapped gate/up or a misplaced scale shows).
* Sampling rows, and exact power-of-two scaling of the down-projection scales.
"""
import math

import numpy as np
import pytest
import torch

from moe_decode_layer_amd import synth
from oracle import moe_oracle as O

SMALL = [
    synth.WORKLOADS[0],
    synth.Workload("t5_h64_e4_k2_s1", T=5, H=64, E=4, K=2, S=1, I=32),
    synth.Workload("t9_h96_e6_k3_s1", T=9, H=96, E=6, K=3, S=1, I=64, zipf_s=1.2),
    synth.Workload("t3_h32_e2_k2_s0", T=3, H=32, E=2, K=2, S=0, I=32),
]


def _torch_dequant(q, s):
    v = torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64)
    return v * torch.from_numpy(s).to(torch.float64).repeat_interleave(32, dim=-1)


def _torch_expert(X, w13, s13, w2, s2):
    I = w13.shape[0] // 2
    W13 = _torch_dequant(w13, s13)
    g = X @ W13[:I].T
    u = X @ W13[I:].T
    h = torch.from_numpy(O.bf16_round((torch.nn.functional.silu(g) * u).numpy()))
    return h @ _torch_dequant(w2, s2).T


def _dense_masked(inp, res):
    wl = inp.workload
    X = torch.from_numpy(O.bf16_bits_to_f64(inp.x))
    y = torch.zeros((wl.T, wl.H), dtype=torch.float64)
    if wl.S:
        y += _torch_expert(X, inp.w13[wl.E], inp.s13[wl.E], inp.w2[wl.E], inp.s2[wl.E])
    mask = torch.zeros((wl.T, wl.E), dtype=torch.float64)
    for t in range(wl.T):
        for k in range(wl.K):
            mask[t, int(res.idx[t, k])] = float(res.w[t, k])
    for e in range(wl.E):
        o = _torch_expert(X, inp.w13[e], inp.s13[e], inp.w2[e], inp.s2[e])
        y += mask[:, e:e + 1] * o
    return y.numpy()


def _inputs(wl):
    inp = synth.make_inputs(wl)
    att = O.choose_attempts(wl, lambda a: synth.x_rows(wl, a), inp.router_w, inp.router_b)
    inp.x = synth.x_rows(wl, att)
    inp.attempts = att
    return inp


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_sparse_equals_dense_masked(wl):
    inp = _inputs(wl)
    res = O.forward(inp)
    dense = _dense_masked(inp, res)
    assert np.abs(res.y - dense).max() <= 1e-12 * np.abs(dense).max()
    assert np.array_equal(res.y_bf16, O.bf16_round(res.y))


def test_single_expert_is_swiglu_mlp():
    wl = synth.Workload("t4_h64_e1_k1_s0", T=4, H=64, E=1, K=1, S=0, I=32)
    inp = synth.make_inputs(wl)
    res = O.forward(inp)
    assert np.all(res.idx == 0) and np.all(res.w == 1.0)
    X = torch.from_numpy(O.bf16_bits_to_f64(inp.x))
    mlp = _torch_expert(X, inp.w13[0], inp.s13[0], inp.w2[0], inp.s2[0]).numpy()
    assert np.array_equal(res.y, mlp)


def test_k_equals_e_is_score_weighted_mixture():
    wl = synth.Workload("t3_h64_e3_k3_s0", T=3, H=64, E=3, K=3, S=0, I=32)
    inp = synth.make_inputs(wl)
    res = O.forward(inp)
    X = torch.from_numpy(O.bf16_bits_to_f64(inp.x))
    s = res.scores / res.scores.sum(axis=1, keepdims=True)
    want = sum(s[:, e:e + 1] * _torch_expert(X, inp.w13[e], inp.s13[e], inp.w2[e], inp.s2[e]).numpy()
               for e in range(3))
    assert np.abs(res.y - want).max() <= 1e-12 * np.abs(want).max()


def test_closed_form_hand_case():
    """T=1, H=32, I=32, E=2, K=1, S=1, x = 0.25 everywhere.

    Router: expert 1 scores higher (logit 1 vs 0) -> idx = [1], w = [1].
    Expert 1: gate rows all 1.0 (scale 1), up rows all 2.0 (code 1.0, scale 2)
      g = 8, u = 16, h = bf16(silu(8) * 16); down rows all 1.0 with scale 0.5
      -> o_n = 0.5 * 32 * h = 16 h.
    Shared expert: gate 0.5, up 1.0 -> g = 4, u = 8, h' = bf16(silu(4) * 8);
      down 1.0 scale 0.25 -> o'_n = 8 h'.
    y = 8 h' + 16 h.
    """
    wl = synth.Workload("hand", T=1, H=32, E=2, K=1, S=1, I=32)
    one = 0x38
    x = np.full((1, 32), 0x3E80, np.uint16)              # bf16 0.25
    Wr = np.zeros((2, 32), np.float32)
    Wr[1, :] = 1.0 / 8                                   # logit 1 for expert 1
    w13 = np.full((3, 64, 32), one, np.uint8)
    s13 = np.ones((3, 64, 1), np.float32)
    s13[1, 32:] = 2.0                                    # expert 1 up rows = 2.0
    s13[2, :32] = 0.5                                    # shared gate rows = 0.5
    w2 = np.full((3, 32, 32), one, np.uint8)
    s2 = np.ones((3, 32, 1), np.float32)
    s2[1] = 0.5
    s2[2] = 0.25
    inp = synth.Inputs(wl, x, Wr, None, w13, s13, w2, s2, np.zeros(1, np.int32))
    res = O.forward(inp)
    assert res.idx.tolist() == [[1]] and res.w.tolist() == [[1.0]]
    silu = lambda v: v / (1.0 + math.exp(-v))
    h = float(O.bf16_round(silu(8.0) * 16.0))
    hs = float(O.bf16_round(silu(4.0) * 8.0))
    want = 8 * hs + 16 * h
    assert np.all(res.y == want)
    assert np.all(res.y_bf16 == O.bf16_round(want))


def test_row_sample_matches_full_run():
    wl = SMALL[2]
    inp = _inputs(wl)
    full = O.forward(inp)
    part = O.forward(inp, rows=[7, 2, 4])
    assert np.array_equal(part.y, full.y[[7, 2, 4]])


def test_power_of_two_down_scales_scale_output_exactly():
    wl = SMALL[1]
    inp = _inputs(wl)
    base = O.forward(inp)
    inp.s2 = inp.s2 * np.float32(4.0)
    scaled = O.forward(inp)
    assert np.array_equal(scaled.y, 4.0 * base.y)
    assert np.array_equal(scaled.y_bf16, 4.0 * base.y_bf16)


@pytest.mark.parametrize("wl", SMALL[1:], ids=lambda w: w.name)
def test_relabelled_experts_change_nothing(wl):
    """Moving routed expert e to id p[e] (its router row, bias and weights
    together) selects p[idx] with the same weights and gives the same y: the
    layer depends on which expert a row picks, not on its number.  Catches an
    expert looked up by its top-k slot, or a router row taken by position."""
    inp = _inputs(wl)
    base = O.forward(inp)
    E = wl.E
    p = np.random.default_rng(11).permutation(E)
    moved = synth.Inputs(wl, inp.x, inp.router_w.copy(), None if inp.router_b is None else inp.router_b.copy(),
                         inp.w13.copy(), inp.s13.copy(), inp.w2.copy(), inp.s2.copy(), inp.attempts)
    moved.router_w[p] = inp.router_w
    if inp.router_b is not None:
        moved.router_b[p] = inp.router_b
    for name in ("w13", "s13", "w2", "s2"):
        getattr(moved, name)[p] = getattr(inp, name)[:E]   # the shared slot E stays
    res = O.forward(moved)
    assert np.array_equal(res.idx, p[base.idx])
    np.testing.assert_allclose(res.w, base.w, rtol=1e-14, atol=0)
    np.testing.assert_allclose(res.y, base.y, rtol=1e-12, atol=1e-12 * np.abs(base.y).max())


@pytest.mark.parametrize("wl", SMALL[1:], ids=lambda w: w.name)
def test_permuted_rows_permute_the_output(wl):
    """Rows are independent: permuting the batch's rows permutes the routing
    and the output rows and changes nothing else (a row's expert outputs are
    never mixed with another row's)."""
    inp = _inputs(wl)
    base = O.forward(inp)
    q = np.random.default_rng(12).permutation(wl.T)
    moved = synth.Inputs(wl, inp.x[q].copy(), inp.router_w, inp.router_b, inp.w13, inp.s13, inp.w2, inp.s2,
                         inp.attempts[q].copy())
    res = O.forward(moved)
    assert np.array_equal(res.idx, base.idx[q])
    np.testing.assert_allclose(res.w, base.w[q], rtol=1e-14, atol=0)
    np.testing.assert_allclose(res.y, base.y[q], rtol=1e-12, atol=1e-12 * np.abs(base.y).max())
    assert np.array_equal(res.placement.count, base.placement.count)
