"""GPU parity of clipped SwiGLU (moe_decode_set_swiglu_limit): every kernel
variant against the oracle with a limit that clips a good share of the gate
and up values, and the default (no clip) restored bit for bit."""
import dataclasses
import json
import math
import os

import numpy as np
import pytest
import torch

from moe_decode_layer_amd import binding, device, synth
from oracle import moe_oracle as O

from block_checks import check_against_plain_run, check_block, run_block
from checks import MAX_REL, MEAN_REL, output_errors

pytestmark = pytest.mark.gpu

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "attempts.json")))


def limit_for(wl):
    """A limit near 1.5 standard deviations of the pre-activations
    (std ~ 0.02 sqrt(H)), rounded to fp32 as the kernel receives it."""
    return float(np.float32(2.0 * math.sqrt(wl.H / 4096)))

BASES = [
    synth.BY_NAME["verify_t6_h4096_e256_k8_s1"],
    synth.BY_NAME["decode_t1_h4096_e256_k8_s1"],
    synth.BY_NAME["tiny_t4_h256_e16_k2"],
    synth.BY_NAME["zipf_t64_h4096_e256_k8_s1"],
    synth.Workload("t9_h4096_e256_k8_s1", T=9, H=4096, E=256, K=8, S=1, I=512),
    synth.Workload("t20_h128_e8_k8_s1", T=20, H=128, E=8, K=8, S=1, I=64),
    synth.Workload("t6_h4096_e256_k8_s1_i576", T=6, H=4096, E=256, K=8, S=1, I=576),
    synth.BY_NAME["zipf_t64_h4096_e256_k8_s1_i576"],      # wide items at I = 576
]


def inputs_for(wl):
    att = GOLDEN["attempts"].get(wl.name)
    if att is None:
        att = O.choose_attempts(wl, lambda a: synth.x_rows(wl, a), synth.router_weights(wl),
                                synth.zipf_bias(wl))
    return synth.make_inputs(wl, att)


@pytest.mark.parametrize("base", BASES, ids=lambda w: w.name)
def test_clipped_swiglu_parity(base):
    print(f"case {base.name} limit {limit_for(base)}", flush=True)
    inp0 = inputs_for(base)
    wl = dataclasses.replace(base, swiglu_limit=limit_for(base))
    inp = dataclasses.replace(inp0, workload=wl)
    ref = O.forward(inp)
    plain = O.forward(inp0)
    # the limit matters: the clipped layer differs from the plain one far
    # beyond the tolerance
    assert output_errors(plain.y_bf16, ref.y_bf16)[0] > 10 * MAX_REL
    layer = device.make_layer(inp)
    out = device.run_once(layer, inp.x, wl.E, wl.K)
    assert np.array_equal(out["topk_idx"], ref.idx)
    assert np.array_equal(out["pair_rank"], ref.placement.rank)
    mx, mean = output_errors(O.bf16_bits_to_f64(out["y"]), ref.y_bf16)
    print(f"{base.name} clipped: max_rel {mx:.3e} mean_rel {mean:.3e}")
    assert mx <= MAX_REL and mean <= MEAN_REL, (mx, mean)
    # back to no clipping: the same bits as a handle that never clipped
    layer.set_swiglu_limit(math.inf)
    again = device.run_once(layer, inp.x, wl.E, wl.K)
    layer.close()
    fresh = device.make_layer(inp0)
    want = device.run_once(fresh, inp0.x, wl.E, wl.K)
    fresh.close()
    assert np.array_equal(again["y"], want["y"])


def test_clip_applies_to_block_runs_and_bad_limits_are_rejected():
    """A clipped block run: routing and xn against the oracle's block, and
    the MoE part held to the layer's max and mean bars through the plain run
    on the kernel's own normalised rows (which clips with the same limit)."""
    base = synth.BY_NAME["verify_t6_h4096_e256_k8_s1_prenorm"]
    wl = dataclasses.replace(base, swiglu_limit=limit_for(base))
    inp = dataclasses.replace(inputs_for(base), workload=wl)
    layer = device.make_layer(inp)
    L = binding.lib()
    for bad in (0.0, -1.0, float("nan")):
        assert L.moe_decode_set_swiglu_limit(layer.handle, bad) == binding.MOE_ERR_INVALID_ARG
    out = run_block(layer, inp, wl)
    check_block(wl, inp, out)
    check_against_plain_run(wl, inp, layer, out)
    layer.close()
    # the clip is in effect in the block run (the unclipped block differs)
    plain_ref = O.forward_block(inputs_for(base))
    assert output_errors(plain_ref.moe.y_bf16, O.forward_block(inp).moe.y_bf16)[0] > 10 * MAX_REL
