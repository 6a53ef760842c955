"""GPU parity of the MX expert weight formats (MXFP4: E2M1 codes, MXFP8:
e4m3fn codes, each with one E8M0 scale per 32 K elements) against the CPU
oracle, at the layer's bars (see test_gpu_parity): routing bit-exact, y
within max|d|/max|o| <= 1e-2 and sum|d|/sum|o| <= 2e-3 on every row.

Every kernel variant an MX handle can take is reached: x in LDS with the
full-tile items (H 4096, I 512, up to 16 rows) and its I = 576 form, x in LDS
with the general items, x in global memory with one and with four MFMA blocks
per item (batches above 16 rows at other shapes), the wide items (batches
above 16 rows at H 4096, I 512: 64 Zipf rows and 384 rows, both formats),
router tiles with distributed top-k, an intermediate width padded from 288 to
320, and pre-norm block runs and clipped SwiGLU on MX weights.
"""
import dataclasses
import json
import math
import os

import numpy as np
import pytest

from block_checks import check_against_plain_run, check_block, run_block
from checks import MAX_REL, MEAN_REL, output_errors
from moe_decode_layer_amd import device, synth
from oracle import moe_oracle as O

from test_gpu_parity import check_against_oracle

pytestmark = pytest.mark.gpu

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "attempts.json")))


def inputs_for(wl):
    att = GOLDEN["attempts"].get(wl.name)
    if att is None:
        att = O.attempts_for(wl, synth.candidate_rows(wl), synth.router_weights(wl),
                             synth.zipf_bias(wl), synth.norm_weight(wl) if wl.prenorm else None)
    return synth.make_inputs(wl, att)


def mx(wl, fmt):
    return dataclasses.replace(wl, name=f"{wl.name}_{fmt}", weight_format=fmt)


@pytest.mark.parametrize("wl", synth.MX, ids=lambda w: w.name)
def test_mx_workload_parity(wl):
    print(f"case {wl.name}", flush=True)
    inp = inputs_for(wl)
    layer = device.make_layer(inp)
    out = device.run_once(layer, inp.x, wl.E, wl.K)
    check_against_oracle(wl, inp, out)
    again = device.run_once(layer, inp.x, wl.E, wl.K)
    assert np.array_equal(again["y"], out["y"])
    layer.close()


EDGE = [
    synth.Workload("t6_h4096_e256_k8_s1_i576", T=6, H=4096, E=256, K=8, S=1, I=576),      # full items, 9 down tiles
    synth.Workload("t6_h4096_e256_k8_s1_i288", T=6, H=4096, E=256, K=8, S=1, I=288),      # padded to 320
    synth.Workload("t9_h4096_e256_k8_s1", T=9, H=4096, E=256, K=8, S=1, I=512),           # x in global memory
    synth.Workload("t64_h4096_e256_k8_s1", T=64, H=4096, E=256, K=8, S=1, I=512, zipf_s=1.2),  # wide items
    synth.Workload("t20_h128_e8_k8_s1", T=20, H=128, E=8, K=8, S=1, I=64),                # router tiles, K = E
    synth.Workload("t70_h192_e4_k2_s1", T=70, H=192, E=4, K=2, S=1, I=192),               # ragged H, 2 chunks, 4 MFMA blocks
    synth.Workload("t3_h64_e1_k1_s0", T=3, H=64, E=1, K=1, S=0, I=64),                    # one expert
]
EDGE_CASES = [mx(w, f) for w in EDGE for f in ("mxfp4", "mxfp8")] + [
    mx(synth.Workload("t384_h4096_e256_k8_s1", T=384, H=4096, E=256, K=8, S=1, I=512), "mxfp4"),
    mx(synth.Workload("t40_h4096_e256_k8_s1_i288", T=40, H=4096, E=256, K=8, S=1, I=288, zipf_s=1.2), "mxfp4"),
]


@pytest.mark.parametrize("wl", EDGE_CASES, ids=lambda w: w.name)
def test_mx_edge_shapes(wl):
    print(f"case {wl.name}", flush=True)
    inp = inputs_for(wl)
    layer = device.make_layer(inp)
    out = device.run_once(layer, inp.x, wl.E, wl.K)
    check_against_oracle(wl, inp, out)
    layer.close()


def test_mx_ragged_T_on_one_handle():
    """One MXFP4 handle for 384 rows run at 384, 17, 64, 1 and 6 rows: the
    wide items above 16 rows and the general ones below, each run against
    the oracle."""
    wl = EDGE_CASES[-2]
    inp = inputs_for(wl)
    layer = device.make_layer(inp, max_tokens=wl.T)
    for T in (384, 17, 64, 1, 6):
        print(f"case {wl.name} T={T}", flush=True)
        sub = synth.Inputs(wl.with_rows(T), inp.x[:T], inp.router_w, inp.router_b, inp.w13,
                           inp.s13, inp.w2, inp.s2, inp.attempts[:T])
        out = device.run_once(layer, np.ascontiguousarray(sub.x), wl.E, wl.K)
        check_against_oracle(sub.workload, sub, out)
    layer.close()


def test_mxfp4_pairs_switch_with_T_on_one_handle():
    """The full-tile MXFP4 kernel takes two row blocks per gate/up item when
    the call can touch enough experts for two such items per workgroup (6 and
    4 rows here) and single row blocks otherwise (1 and 3 rows): one 6-row
    handle run at 6, 1, 4, 3 and 6 rows, each run against the oracle."""
    wl = synth.BY_NAME["verify_t6_h4096_e256_k8_s1_mxfp4"]
    inp = inputs_for(wl)
    layer = device.make_layer(inp, max_tokens=wl.T)
    for T in (6, 1, 4, 3, 6):
        print(f"case {wl.name} T={T}", flush=True)
        sub = synth.Inputs(wl.with_rows(T), inp.x[:T], inp.router_w, inp.router_b, inp.w13,
                           inp.s13, inp.w2, inp.s2, inp.attempts[:T])
        out = device.run_once(layer, np.ascontiguousarray(sub.x), wl.E, wl.K)
        check_against_oracle(sub.workload, sub, out)
    layer.close()


BLOCK_CASES = [dataclasses.replace(w, name=w.name + "_prenorm", prenorm=True) for w in (
    mx(synth.BY_NAME["verify_t6_h4096_e256_k8_s1"], "mxfp4"),
    mx(synth.BY_NAME["verify_t6_h4096_e256_k8_s1"], "mxfp8"),
    mx(synth.Workload("t9_h4096_e256_k8_s1", T=9, H=4096, E=256, K=8, S=1, I=512), "mxfp4"),
    mx(synth.Workload("t33_h320_e64_k6_s1", T=33, H=320, E=64, K=6, S=1, I=128, zipf_s=1.2), "mxfp8"),
)]


@pytest.mark.parametrize("wl", BLOCK_CASES, ids=lambda w: w.name)
def test_mx_block_parity(wl):
    print(f"case {wl.name}", flush=True)
    inp = inputs_for(wl)
    layer = device.make_layer(inp)
    out = run_block(layer, inp, wl)
    check_block(wl, inp, out)
    check_against_plain_run(wl, inp, layer, out)
    layer.close()


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_mx_clipped_swiglu_parity(fmt):
    base = synth.BY_NAME[f"verify_t6_h4096_e256_k8_s1_{fmt}"]
    inp0 = inputs_for(base)
    wl = dataclasses.replace(base, swiglu_limit=float(np.float32(2.0)))
    print(f"case {wl.name} limit {wl.swiglu_limit}", flush=True)
    inp = dataclasses.replace(inp0, workload=wl)
    ref = O.forward(inp)
    assert output_errors(O.forward(inp0).y_bf16, ref.y_bf16)[0] > 10 * MAX_REL   # the limit bites
    layer = device.make_layer(inp)
    out = device.run_once(layer, inp.x, wl.E, wl.K)
    assert np.array_equal(out["topk_idx"], ref.idx)
    mx_, mean = output_errors(O.bf16_bits_to_f64(out["y"]), ref.y_bf16)
    print(f"{wl.name} clipped: max_rel {mx_:.3e} mean_rel {mean:.3e}")
    assert mx_ <= MAX_REL and mean <= MEAN_REL, (mx_, mean)
    layer.set_swiglu_limit(math.inf)
    layer.close()


def test_formats_give_different_layers_on_the_same_normals():
    """The three formats quantise the same normal draws: their outputs agree
    roughly (the layer computes the same function of nearly the same weights)
    but not exactly (each format's rounding is its own), which shows the
    handle really decodes the format it was created with."""
    ys = {}
    for fmt in ("fp8", "mxfp8", "mxfp4"):
        name = "verify_t6_h4096_e256_k8_s1" + ("" if fmt == "fp8" else f"_{fmt}")
        wl = synth.BY_NAME[name]
        inp = inputs_for(wl)
        layer = device.make_layer(inp)
        ys[fmt] = O.bf16_bits_to_f64(device.run_once(layer, inp.x, wl.E, wl.K, debug=False)["y"])
        layer.close()
    scale = np.abs(ys["fp8"]).max()
    for a, b in (("fp8", "mxfp8"), ("fp8", "mxfp4"), ("mxfp8", "mxfp4")):
        d = np.abs(ys[a] - ys[b]).max() / scale
        print(f"{a} vs {b}: max rel {d:.3e}")
        assert 0 < d < 0.5, (a, b, d)
