"""Pins of the oracle's pre-norm block: the input RMSNorm and the residual add.

RMSNorm is checked against a worked example computed by hand, constant rows,
its scale invariance, a power-of-two change of the weight, its mean-square
property and torch's own rms_norm in fp64; the residual add against the
special case of all-zero experts (the block then returns its input exactly).
"""
import dataclasses

import numpy as np
import torch

from moe_decode_layer_amd import synth
from oracle import moe_oracle as O


def bits(values):
    return O.bf16_value_to_bits(np.asarray(values, np.float64))


def test_worked_example():
    # x = [3, 4, 0, 0]: mean square 25/4, root 2.5, so x / rms = [1.2, 1.6, 0, 0];
    # weight [1, 0.5, 2, 1] gives [1.2, 0.8, 0, 0].  bf16 keeps 8 significant
    # bits: 1.2 = 1.0011001 1001..b rounds up to 1.0011010b = 1.203125 (0x3F9A),
    # 0.8 = 1.1001100 1100..b x 2^-1 rounds up to 0.80078125 (0x3F4D).
    x = np.array([[0x4040, 0x4080, 0x0000, 0x0000]], np.uint16)
    got = O.rmsnorm_bf16(x, np.array([1.0, 0.5, 2.0, 1.0]), 0.0)
    assert got.tolist() == [[0x3F9A, 0x3F4D, 0x0000, 0x0000]]


def test_constant_rows_normalise_to_the_weight():
    # every element c: c / sqrt(c^2 + eps) = 1 - O(eps / c^2), which rounds to 1.0
    for c in (3.0, -0.5, 96.0):
        x = np.full((2, 64), bits([c])[0], np.uint16)
        got = O.rmsnorm_bf16(x, np.ones(64), 1e-6)
        assert np.all(got == bits([np.sign(c)])[0])


def test_epsilon_inside_the_root():
    # x = 2^-12 everywhere, eps = 3 * 2^-24: mean square + eps = 2^-22, root
    # 2^-11, so every output is exactly 0.5 (without eps it would be 1.0)
    x = np.full((1, 128), bits([2.0 ** -12])[0], np.uint16)
    got = O.rmsnorm_bf16(x, np.ones(128), 3.0 * 2.0 ** -24)
    assert np.all(got == bits([0.5])[0])


def test_scale_invariance_and_weight_scaling():
    rng = np.random.default_rng(3)
    x = bits(O.bf16_round(rng.standard_normal((5, 256))))
    g = rng.uniform(0.5, 1.5, 256)
    base = O.rmsnorm_bf16(x, g, 0.0)
    for k in (-3, 1, 7):
        xs = bits(O.bf16_bits_to_f64(x) * 2.0 ** k)
        assert np.array_equal(O.rmsnorm_bf16(xs, g, 0.0), base), k
    # a power-of-two weight scales the output exactly (rounding commutes with it)
    doubled = O.bf16_bits_to_f64(O.rmsnorm_bf16(x, 2.0 * g, 0.0))
    assert np.array_equal(doubled, 2.0 * O.bf16_bits_to_f64(base))


def test_unit_mean_square():
    rng = np.random.default_rng(4)
    x = bits(O.bf16_round(3.0 * rng.standard_normal((8, 4096))))
    y = O.bf16_bits_to_f64(O.rmsnorm_bf16(x, np.ones(4096), 1e-6))
    ms = np.mean(y * y, axis=1)
    # each element carries a relative rounding error below 2^-8
    assert np.all(np.abs(ms - 1.0) < 2.0 ** -7)


def test_matches_torch_rms_norm():
    rng = np.random.default_rng(5)
    H = 1024
    x = bits(O.bf16_round(rng.standard_normal((16, H)) * rng.uniform(0.1, 10, (16, 1))))
    g = 1.0 + 0.1 * rng.standard_normal(H)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(O.bf16_bits_to_f64(x)), (H,),
                                       torch.from_numpy(g), eps=1e-6).numpy()
    got = O.bf16_bits_to_f64(O.rmsnorm_bf16(x, g, 1e-6))
    assert np.array_equal(got, O.bf16_round(ref))


def test_zero_experts_return_the_block_input():
    wl = dataclasses.replace(synth.BY_NAME["tiny_t4_h256_e16_k2_prenorm"], S=1)
    inp = synth.make_inputs(wl)
    zero = dataclasses.replace(inp, w13=np.zeros_like(inp.w13), w2=np.zeros_like(inp.w2))
    res = O.forward_block(zero)
    assert np.array_equal(bits(res.y_bf16), inp.x)
    # the layer still routed the normalised rows
    assert res.moe.idx.shape == (wl.T, wl.K)
    ref = O.router_logits(O.bf16_bits_to_f64(res.xn), inp.router_w, inp.router_b)
    assert np.array_equal(res.moe.logits, ref)


def test_block_rows_recipe():
    wl = synth.BY_NAME["verify_t6_h4096_e256_k8_s1_prenorm"]
    att = np.arange(wl.T, dtype=np.int32) % 2
    plain = O.bf16_bits_to_f64(synth.x_rows(wl, att))
    block = O.bf16_bits_to_f64(synth.block_rows(wl, att))
    for t in range(wl.T):
        assert np.array_equal(block[t], plain[t] * 2.0 ** (t % 3 - 1))
    g = synth.norm_weight(wl)
    assert g.dtype == np.float32 and abs(float(g.mean()) - 1.0) < 0.01
    assert 0.08 < float(g.std()) < 0.12


def test_residual_is_rounded_once():
    # x = 1, moe = 2^-8 + 2^-16: the exact sum lies just above the midpoint
    # 1 + 2^-8 between the bf16 neighbours 1 and 1 + 2^-7, so one rounding
    # gives 1 + 2^-7.  Rounding moe first (to 2^-8, a tie resolved to even)
    # and then the sum (the midpoint, a tie resolved to even) would give 1.
    x = bits([[1.0, -1.0, 4.0]])
    moe = np.array([[2.0 ** -8 + 2.0 ** -16, -(2.0 ** -8 + 2.0 ** -16), 2.0 ** -6 + 2.0 ** -14]])
    got = O.residual_add(x, moe)
    assert got.tolist() == [[1.0 + 2.0 ** -7, -(1.0 + 2.0 ** -7), 4.0 + 2.0 ** -5]]
    double = O.bf16_round(O.bf16_bits_to_f64(x) + O.bf16_round(moe))
    assert double.tolist() == [[1.0, -1.0, 4.0]]


def test_block_output_uses_the_single_rounding():
    # forward_block's y_bf16 is residual_add of its own x and unrounded moe
    wl = synth.BY_NAME["tiny_t4_h256_e16_k2_prenorm"]
    inp = synth.make_inputs(wl)
    res = O.forward_block(inp)
    assert np.array_equal(res.y_bf16, O.residual_add(inp.x, res.moe.y))
    assert np.array_equal(res.y, O.bf16_bits_to_f64(inp.x) + res.moe.y)
