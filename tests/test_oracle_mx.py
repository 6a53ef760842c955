"""Pins of the oracle's MX expert-weight formats: MXFP4 and MXFP8 with one
E8M0 scale per 32 contiguous K elements (OCP Microscaling formats), the
pages' MoE weight formats ("Beyond Day-0: Optimizing DeepSeek-V4.1 Flash in
SGLang", section 3.1: Marlin MoE with MXFP4 weights and BF16 activations;
section 2.1: group32 FP8 reorganised for MXFP8 kernels).

* E8M0: every code against torch's float8_e8m0fnu decoder (0xFF is NaN).
* E2M1: every code against the specification's value table
  (tests/golden/e2m1_values.txt).
* MXFP4 against MXFP8: the E2M1 values re-encoded by torch's own e4m3fn
  encoder decode, as MXFP8 with the same scales, to the same matrix; this
  pins the nibble order and the scale blocks through a second decoder.
* Scale blocks: block b's scale reaches K [32 b, 32 b + 32) and nothing else.
* Expert FFN: sparse = dense masked evaluation with torch's decoders, one
  expert = a SwiGLU MLP, and E8M0 codes raised by 2 on the down projection
  scale y by 4 exactly.
* The input generator's MX quantiser: each block's scale is the largest
  power of two that keeps the block maximum within the element range's top
  binade, elements saturate, and dequantised weights stay within half an
  element step of the drawn normals.
"""
import os

import numpy as np
import pytest
import torch

from moe_decode_layer_amd import synth
from oracle import moe_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def e2m1_table():
    vals = {}
    for line in open(os.path.join(HERE, "golden", "e2m1_values.txt")):
        if line.strip() and not line.startswith("#"):
            c, v = line.split()
            vals[int(c)] = float(v)
    assert sorted(vals) == list(range(16))
    return np.array([vals[c] for c in range(16)])


def torch_e8m0(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e8m0fnu)
    return t.to(torch.float64)


def torch_dequant(q, s, fmt):
    """The same dequantisation with torch's decoders (independent of the oracle's)."""
    scale = torch_e8m0(s).repeat_interleave(32, dim=-1)
    if fmt == "mxfp8":
        v = torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64)
    else:
        tab = torch.from_numpy(e2m1_table())
        b = torch.from_numpy(np.ascontiguousarray(q).astype(np.int64))
        v = tab[torch.stack([b & 0xF, b >> 4], dim=-1).reshape(*b.shape[:-1], 2 * b.shape[-1])]
    return v * scale


def test_e8m0_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    want = torch_e8m0(codes).numpy()
    assert np.isnan(O.E8M0[255]) and np.isnan(want[255])
    assert np.array_equal(O.E8M0[:255], want[:255])
    assert O.E8M0[127] == 1.0 and O.E8M0[0] == 2.0 ** -127 and O.E8M0[254] == 2.0 ** 127


def test_e2m1_matches_the_specification_table():
    tab = e2m1_table()
    assert np.array_equal(O.E2M1, tab)
    assert np.array_equal(np.signbit(O.E2M1), np.signbit(tab))


def test_mxfp4_equals_mxfp8_of_the_same_values():
    rng = np.random.default_rng(0)
    q4 = rng.integers(0, 256, size=(5, 64), dtype=np.uint8)           # K = 128
    s = rng.integers(100, 140, size=(5, 4), dtype=np.uint8)
    codes = np.stack([q4 & 0xF, q4 >> 4], axis=-1).reshape(5, 128)
    # torch encodes each E2M1 value as e4m3fn (exactly representable)
    vals = torch.from_numpy(e2m1_table()[codes])
    q8 = vals.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.dequant(q4, s, "mxfp4"), O.dequant(q8, s, "mxfp8"))
    assert np.array_equal(O.dequant(q4, s, "mxfp4"), torch_dequant(q4, s, "mxfp4").numpy())
    assert np.array_equal(O.dequant(q8, s, "mxfp8"), torch_dequant(q8, s, "mxfp8").numpy())


def test_nibble_order_and_scale_blocks():
    # byte 0x21: element 0 = code 1 (0.5), element 1 = code 2 (1.0)
    q = np.zeros((1, 32), np.uint8)
    q[0, 0] = 0x21
    q[0, 16] = 0x7F                                      # elements 32, 33: code 15 (-6), code 7 (6)
    s = np.array([[127, 129]], np.uint8)                 # scales 1 and 4
    w = O.dequant(q, s, "mxfp4")
    assert w.shape == (1, 64)
    assert w[0, 0] == 0.5 and w[0, 1] == 1.0
    assert w[0, 32] == -24.0 and w[0, 33] == 24.0
    assert np.count_nonzero(w) == 4
    q8 = np.zeros((1, 64), np.uint8)
    q8[0, 31] = 0x38                                     # e4m3fn 1.0 at the last K of block 0
    q8[0, 32] = 0x38                                     # and the first of block 1
    w8 = O.dequant(q8, s, "mxfp8")
    assert w8[0, 31] == 1.0 and w8[0, 32] == 4.0 and np.count_nonzero(w8) == 2


MXSMALL = [synth.Workload("t5_h64_e4_k2_s1", T=5, H=64, E=4, K=2, S=1, I=32),
           synth.Workload("t9_h96_e6_k3_s1", T=9, H=96, E=6, K=3, S=1, I=64, zipf_s=1.2)]


def _torch_expert(X, w13, s13, w2, s2, fmt):
    I = w13.shape[0] // 2
    W13 = torch_dequant(w13, s13, fmt)
    g = X @ W13[:I].T
    u = X @ W13[I:].T
    h = torch.from_numpy(O.bf16_round((torch.nn.functional.silu(g) * u).numpy()))
    return h @ torch_dequant(w2, s2, fmt).T


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("base", MXSMALL, ids=lambda w: w.name)
def test_sparse_equals_dense_masked(base, fmt):
    import dataclasses
    wl = dataclasses.replace(base, weight_format=fmt)
    inp = synth.make_inputs(wl)
    att = O.choose_attempts(wl, lambda a: synth.x_rows(wl, a), inp.router_w, inp.router_b)
    inp.x = synth.x_rows(wl, att)
    res = O.forward(inp)
    X = torch.from_numpy(O.bf16_bits_to_f64(inp.x))
    y = torch.zeros((wl.T, wl.H), dtype=torch.float64)
    if wl.S:
        y += _torch_expert(X, inp.w13[wl.E], inp.s13[wl.E], inp.w2[wl.E], inp.s2[wl.E], fmt)
    for e in range(wl.E):
        m = torch.zeros((wl.T, 1), dtype=torch.float64)
        for t in range(wl.T):
            for k in range(wl.K):
                if res.idx[t, k] == e:
                    m[t, 0] = float(res.w[t, k])
        y += m * _torch_expert(X, inp.w13[e], inp.s13[e], inp.w2[e], inp.s2[e], fmt)
    assert np.abs(res.y - y.numpy()).max() <= 1e-12 * np.abs(y.numpy()).max()


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_single_expert_is_swiglu_mlp_and_scales_are_exact(fmt):
    wl = synth.Workload("t4_h64_e1_k1_s0", T=4, H=64, E=1, K=1, S=0, I=32, weight_format=fmt)
    inp = synth.make_inputs(wl)
    res = O.forward(inp)
    X = torch.from_numpy(O.bf16_bits_to_f64(inp.x))
    mlp = _torch_expert(X, inp.w13[0], inp.s13[0], inp.w2[0], inp.s2[0], fmt).numpy()
    assert np.array_equal(res.y, mlp)
    inp.s2 = (inp.s2.astype(np.int32) + 2).astype(np.uint8)        # every down scale x 4
    assert np.array_equal(O.forward(inp).y, 4.0 * res.y)


@pytest.mark.parametrize("fmt,emax,top", [("mxfp4", 2, 6.0), ("mxfp8", 8, 448.0)])
def test_generator_mx_quantiser(fmt, emax, top):
    wl = synth.Workload("q", T=1, H=256, E=1, K=1, S=0, I=64, weight_format=fmt)
    w13, s13, w2, s2 = synth.expert_weights(wl)
    W = O.dequant(w13[0], s13[0], fmt)                                # [2I][H]
    rows = [synth.normals(wl.seed, synth.TENSOR_W13, 0, r, wl.H) * wl.expert_std for r in range(2 * wl.I)]
    ref = np.stack(rows)
    X = s13[0].astype(np.int64) - 127                                  # block exponents
    amax = np.abs(ref.reshape(2 * wl.I, -1, 32)).max(axis=2)
    assert np.array_equal(X, np.floor(np.log2(amax)).astype(np.int64) - emax)
    elem = (W / np.repeat(2.0 ** X, 32, axis=1))
    assert np.abs(elem).max() <= top
    # away from saturation, within half a step of the element grid
    step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30) / np.repeat(2.0 ** X, 32, axis=1)))
                   - (1 if fmt == "mxfp4" else 3))
    ok = np.abs(ref) / np.repeat(2.0 ** X, 32, axis=1) < top
    err = np.abs(W - ref) / np.repeat(2.0 ** X, 32, axis=1)
    assert np.all(err[ok] <= np.maximum(step[ok], 2.0 ** (-1 if fmt == "mxfp4" else -9)) / 2 + 1e-12)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_relabelled_experts_change_nothing(fmt):
    """MX weights moved with their expert to a permuted id (codes and E8M0
    scales together) give the same selections, mapped, and the same y."""
    import dataclasses
    wl = dataclasses.replace(MXSMALL[1], weight_format=fmt)
    inp = synth.make_inputs(wl)
    att = O.choose_attempts(wl, lambda a: synth.x_rows(wl, a), inp.router_w, inp.router_b)
    inp.x = synth.x_rows(wl, att)
    base = O.forward(inp)
    p = np.random.default_rng(13).permutation(wl.E)
    moved = synth.Inputs(wl, inp.x, inp.router_w.copy(), inp.router_b.copy(), inp.w13.copy(),
                         inp.s13.copy(), inp.w2.copy(), inp.s2.copy(), att)
    moved.router_w[p] = inp.router_w
    moved.router_b[p] = inp.router_b
    for name in ("w13", "s13", "w2", "s2"):
        getattr(moved, name)[p] = getattr(inp, name)[:wl.E]
    res = O.forward(moved)
    assert np.array_equal(res.idx, p[base.idx])
    np.testing.assert_allclose(res.y, base.y, rtol=1e-12, atol=1e-12 * np.abs(base.y).max())
