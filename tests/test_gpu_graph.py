"""Runs captured in a HIP graph and replayed.

The run's tag and counter block come from arrival counters in device memory
that every launch advances, so a captured launch replays correctly.  Three
plain and three block calls on one handle are captured in one graph and the
graph is replayed 20 times.  Between replays the inputs are rewritten in
place (two row rotations in turn), the outputs are overwritten, and eager
runs of the same handle are interleaved; every replay's outputs must equal,
bit for bit, the eager run on the same rows, which is itself checked against
the oracle.
"""
import dataclasses
import json
import os

import numpy as np
import pytest
import torch

from block_checks import check_block, rolled, run_block
from checks import MAX_REL, MEAN_REL, output_errors
from moe_decode_layer_amd import binding, device, synth
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "attempts.json")))


def _bits(t):
    return t.cpu().numpy().view(np.uint16)


def _inputs(wl):
    att = GOLDEN["attempts"].get(wl.name)
    if att is None:
        att = O.attempts_for(wl, synth.candidate_rows(wl), synth.router_weights(wl),
                             synth.zipf_bias(wl), synth.norm_weight(wl))
    return synth.make_inputs(wl, att)


CASES = [synth.BY_NAME["verify_t6_h4096_e256_k8_s1_prenorm"],
         synth.BY_NAME["verify_t384_h4096_e256_k8_s1_prenorm"],
         # MXFP4 weights: the full-tile kernel with two row blocks per gate/up item
         dataclasses.replace(synth.BY_NAME["verify_t6_h4096_e256_k8_s1_mxfp4"],
                             name="verify_t6_h4096_e256_k8_s1_mxfp4_prenorm", prenorm=True)]


@pytest.mark.parametrize("wl", CASES, ids=["t6", "t384", "t6_mxfp4"])
def test_graph_replays_match_eager_runs(wl):
    name = wl.name
    print(f"case graph replay {name}", flush=True)
    inp = _inputs(wl)
    layer = device.make_layer(inp)
    dev = torch.device("cuda", 0)
    sets = []
    for shift in (0, 1):
        blk = rolled(inp, shift)
        # plain runs take the normalised rows (their routing margins hold)
        xn = O.rmsnorm_bf16(blk.x, inp.norm_w, wl.norm_eps)
        plain = dataclasses.replace(blk, workload=dataclasses.replace(wl, prenorm=False), x=xn)
        out_p = device.run_once(layer, xn, wl.E, wl.K)
        ref = O.forward(plain)
        assert np.array_equal(out_p["topk_idx"], ref.idx)
        mx, mean = output_errors(O.bf16_bits_to_f64(out_p["y"]), ref.y_bf16)
        assert mx <= MAX_REL and mean <= MEAN_REL, (mx, mean)
        out_b = run_block(layer, blk, wl)
        check_block(wl, blk, out_b)
        sets.append((xn, blk.x, out_p["y"], out_b["y"]))

    xp = device.to_device(sets[0][0], dev)
    xb = device.to_device(sets[0][1], dev)
    yp = [torch.empty_like(xp) for _ in range(3)]
    yb = [torch.empty_like(xb) for _ in range(3)]
    # one eager call of each kind on these buffers first (the library caches
    # its occupancy query outside the capture)
    layer.run(xp, yp[0])
    layer.run_block(xb, yb[0])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(3):
            layer.run(xp, yp[i])
            layer.run_block(xb, yb[i])
    # eager work between replays: a run on separate buffers
    x_e = device.to_device(sets[1][0], dev)
    y_e = torch.empty_like(x_e)
    for r in range(20):
        k = r % 2
        xp.copy_(device.to_device(sets[k][0], dev))
        xb.copy_(device.to_device(sets[k][1], dev))
        for t in yp + yb:
            t.fill_(-1)
        g.replay()
        layer.run(x_e, y_e)
        torch.cuda.synchronize()
        assert layer.check() == binding.MOE_OK, f"replay {r}"
        for i in range(3):
            assert np.array_equal(_bits(yp[i]), sets[k][2]), f"replay {r}: plain call {i} differs"
            assert np.array_equal(_bits(yb[i]), sets[k][3]), f"replay {r}: block call {i} differs"
        assert np.array_equal(_bits(y_e), sets[1][2]), f"eager run after replay {r} differs"
    del g
    layer.close()
