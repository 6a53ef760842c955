"""Pins of the oracle's clipped SwiGLU: a hand-computed value, the bound the
clip implies, and no change for a limit above every pre-activation."""
import dataclasses
import math

import numpy as np

from moe_decode_layer_amd import synth
from oracle import moe_oracle as O


def one_expert(g, u, I=32, H=32):
    """One expert whose gate row 0 and up row 0 read x[0] with weights g and u
    (exact in e4m3fn with scale 1), and whose down row 0 reads h[0] with weight 1."""
    code = {v: c for c, v in enumerate(O.E4M3FN) if not math.isnan(v)}
    w13 = np.zeros((2 * I, H), np.uint8)
    w13[0, 0] = code[g]
    w13[I, 0] = code[u]
    s13 = np.ones((2 * I, H // 32), np.float32)
    w2 = np.zeros((H, I), np.uint8)
    w2[0, 0] = code[1.0]
    s2 = np.ones((H, I // 32), np.float32)
    X = np.zeros((1, H))
    X[0, 0] = 1.0
    return X, w13, s13, w2, s2


def test_hand_computed_clip():
    # g = 5, u = -7, L = 2: silu(2) * (-2) = -4 / (1 + e^-2) = -3.52318831...; bf16
    # spacing at 3.5 is 2^-6, and -225.48 steps rounds to -225: h = -3.515625
    X, w13, s13, w2, s2 = one_expert(5.0, -7.0)
    o = O.expert_ffn(X, w13, s13, w2, s2, limit=2.0)
    assert o[0, 0] == -3.515625
    assert np.all(o[0, 1:] == 0.0)
    # no limit: silu(5) * (-7) = -34.7658...; spacing 2^-2 at 32: -34.75
    assert O.expert_ffn(X, w13, s13, w2, s2)[0, 0] == -34.75


def test_gate_is_capped_from_above_only():
    # g = -6 stays -6 under L = 2: silu(-6) * 1.5 = -0.0222...; bf16 -0.022216796875
    X, w13, s13, w2, s2 = one_expert(-6.0, 1.5)
    got = O.expert_ffn(X, w13, s13, w2, s2, limit=2.0)[0, 0]
    assert got == O.expert_ffn(X, w13, s13, w2, s2)[0, 0]
    assert abs(got - (-6.0 / (1.0 + math.exp(6.0)) * 1.5)) < 2.0 ** -13


def test_clip_bounds_h_and_large_limits_change_nothing():
    wl = dataclasses.replace(synth.BY_NAME["tiny_t4_h256_e16_k2"], S=1)
    inp = synth.make_inputs(wl)
    X = O.bf16_bits_to_f64(inp.x)
    W13 = O.dequant(inp.w13[0], inp.s13[0])
    I = W13.shape[0] // 2
    pre = np.abs(X @ W13.T).max()
    base = O.expert_ffn(X, inp.w13[0], inp.s13[0], inp.w2[0], inp.s2[0])
    assert np.array_equal(O.expert_ffn(X, inp.w13[0], inp.s13[0], inp.w2[0], inp.s2[0],
                                       limit=2 * pre), base)
    # with L = 0.25 every |h| <= max(silu(L), 0.279) * L, so |o| <= that * sum |W2 row|
    L = 0.25
    o = O.expert_ffn(X, inp.w13[0], inp.s13[0], inp.w2[0], inp.s2[0], limit=L)
    W2 = O.dequant(inp.w2[0], inp.s2[0])
    bound = max(L / (1 + math.exp(-L)), 0.2785) * L * 1.01 * np.abs(W2).sum(axis=1)
    assert np.all(np.abs(o) <= bound[None, :])
    assert not np.array_equal(o, base)


def test_forward_uses_the_workload_limit():
    wl = synth.BY_NAME["tiny_t4_h256_e16_k2"]
    inp = synth.make_inputs(wl)
    clipped = dataclasses.replace(inp, workload=dataclasses.replace(wl, swiglu_limit=0.1))
    a, b = O.forward(inp), O.forward(clipped)
    assert np.array_equal(a.idx, b.idx) and not np.array_equal(a.y, b.y)
