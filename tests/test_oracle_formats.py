"""Pins of the oracle's number formats: FP8 e4m3fn decoding and bf16 rounding.

e4m3fn is checked against torch's float8_e4m3fn decoder (an independent
library implementation of the OCP FP8 format) over all 256 codes, plus spot
values of the format; bf16 rounding against torch's fp32 -> bf16 conversion
and textbook round-to-nearest-even vectors, including the cases where
rounding through fp32 first would give a different answer.
"""
import math

import numpy as np
import torch

from oracle import moe_oracle as O


def test_e4m3fn_matches_library_decoder_on_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = O.E4M3FN
    nan = np.isnan(lib)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ours[~nan], lib[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(lib[~nan]))


def test_e4m3fn_spot_values():
    assert O.E4M3FN[0x38] == 1.0
    assert O.E4M3FN[0x7E] == 448.0
    assert O.E4M3FN[0xFE] == -448.0
    assert O.E4M3FN[0x08] == 2.0 ** -6       # smallest normal
    assert O.E4M3FN[0x07] == 7 * 2.0 ** -9   # largest subnormal
    assert O.E4M3FN[0x01] == 2.0 ** -9       # smallest subnormal
    assert O.E4M3FN[0x00] == 0.0 and O.E4M3FN[0x80] == 0.0
    assert math.isnan(O.E4M3FN[0x7F]) and math.isnan(O.E4M3FN[0xFF])
    finite = O.E4M3FN[~np.isnan(O.E4M3FN)]
    assert finite.size == 254
    pos = O.E4M3FN[:0x7F]
    assert np.all(np.diff(pos) > 0)           # codes 0..0x7E increase strictly


def test_dequant_applies_one_scale_per_32_k():
    q = np.full((2, 64), 0x38, np.uint8)      # all 1.0
    s = np.array([[0.5, 4.0], [2.0 ** -20, 3.0]], np.float32)
    d = O.dequant(q, s)
    assert np.all(d[0, :32] == 0.5) and np.all(d[0, 32:] == 4.0)
    assert np.all(d[1, :32] == 2.0 ** -20) and np.all(d[1, 32:] == 3.0)


def test_bf16_bits_roundtrip():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    v = O.bf16_bits_to_f64(bits)
    fin = np.isfinite(v)
    back = O.bf16_value_to_bits(v[fin])
    assert np.array_equal(back, bits[fin])


def test_bf16_round_matches_library_on_fp32_values():
    rng = np.random.default_rng(0)
    f = np.concatenate([
        rng.standard_normal(50000).astype(np.float32),
        (rng.standard_normal(5000) * 1e-39).astype(np.float32),
        (rng.standard_normal(5000) * 1e38).astype(np.float32),
    ])
    lib = torch.from_numpy(f).to(torch.bfloat16).to(torch.float64).numpy()
    ours = O.bf16_round(f.astype(np.float64))
    assert np.array_equal(ours, lib)


def test_bf16_round_textbook_vectors():
    r = O.bf16_round
    assert r(1.0 + 2.0 ** -8) == 1.0                       # tie -> even (down)
    assert r(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6       # tie -> even (up)
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7  # direct from fp64: just above the tie
    assert r(-(1.0 + 2.0 ** -8 + 2.0 ** -30)) == -(1.0 + 2.0 ** -7)
    assert r(O.BF16_MAX) == O.BF16_MAX
    assert r(O.BF16_MAX + 2.0 ** 119) == math.inf          # exactly half a step above max
    assert r(O.BF16_MAX + 2.0 ** 118) == O.BF16_MAX
    assert r(2.0 ** -133) == 2.0 ** -133                   # smallest subnormal
    assert r(2.0 ** -134) == 0.0                           # tie -> even (zero)
    assert r(3 * 2.0 ** -134) == 2.0 ** -132               # tie -> even (2 steps)
    assert r(0.0) == 0.0
    # fp32 double rounding would give 1.0 for the first of these
    v32 = np.float32(1.0 + 2.0 ** -8 + 2.0 ** -30)
    assert float(torch.tensor(float(v32)).to(torch.bfloat16)) == 1.0


def test_sigmoid_special_values():
    s = O.sigmoid(np.array([0.0, 1000.0, -1000.0, math.log(3.0)]))
    assert s[0] == 0.5 and s[1] == 1.0 and s[2] == 0.0
    assert abs(s[3] - 0.75) < 1e-15
