"""GPU parity of the pre-norm block runs (moe_decode_run_block): input RMSNorm
in the kernel's prologue, the layer on the normalised rows, the residual added
in the combine.  Checked against the oracle's block (fp64) and against the
plain layer run on the kernel's own normalised rows.
"""
import dataclasses
import json
import os

import numpy as np
import pytest
import torch

from moe_decode_layer_amd import binding, device, synth
from oracle import moe_oracle as O

from checks import MAX_REL, MEAN_REL, check_placement

pytestmark = pytest.mark.gpu

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "attempts.json")))


def block_of(wl):
    return dataclasses.replace(wl, name=wl.name + "_prenorm", prenorm=True)


def inputs_for(wl):
    att = GOLDEN["attempts"].get(wl.name)
    if att is None:
        att = O.attempts_for(wl, synth.candidate_rows(wl), synth.router_weights(wl),
                             synth.zipf_bias(wl), synth.norm_weight(wl))
    return synth.make_inputs(wl, att)


def bf16_half_ulp(v):
    """Half the bf16 spacing at |v| (the largest rounding error of v)."""
    _, e = np.frexp(np.abs(v))
    return np.ldexp(1.0, np.maximum(e - 8, -133) - 1)


def check_block(wl, inp, out, rows=None):
    """The kernel's normalised rows, routing and output against the oracle."""
    ref = O.forward_block(inp, rows)
    # xn: fp32 in the kernel, fp64 in the oracle, so an element whose exact
    # value lies within a few fp32 steps of a bf16 rounding midpoint may round
    # the other way: at most one bf16 step, on a small fraction of elements
    got = O.bf16_bits_to_f64(out["norm_x"])
    want = O.bf16_bits_to_f64(ref.xn)
    off = got != want
    assert np.all(np.abs(got - want)[off] <= 2 * bf16_half_ulp(want)[off]), "xn differs by more than one step"
    assert off.mean() <= 1e-3, f"xn: {off.mean():.2e} of elements differ"
    m = ref.moe
    assert np.array_equal(out["topk_idx"], m.idx), "top-k indices differ"
    assert np.array_equal(out["expert_count"], m.placement.count)
    assert np.array_equal(out["pair_rank"], m.placement.rank)
    check_placement(out["topk_idx"], out["pair_rank"], out["expert_count"], wl.E)
    assert np.abs(out["topk_w"] - m.w).max() <= 1e-5
    # the router ran on the kernel's xn (pinned above to one step of the
    # oracle's): its logits are held to the layer's bar against the oracle's
    # router on those same rows
    ref_l = O.router_logits(got, inp.router_w, inp.router_b)
    l_err = np.abs(out["logits"] - ref_l).max() / np.abs(ref_l).max()
    assert l_err <= 1e-4, f"logits rel err {l_err}"
    # y = bf16(x + moe): the kernel's y less the exact block output is its own
    # rounding (half a step of y) plus the layer's error, held to the layer's
    # bar relative to the MoE output (max and mean)
    y = O.bf16_bits_to_f64(out["y"])[ref.moe.rows]
    err = np.abs(y - ref.y) - bf16_half_ulp(y)
    mx = max(float(err.max()), 0.0) / np.abs(m.y).max()
    mean = max(float(np.abs(y - ref.y).mean() - bf16_half_ulp(y).mean()), 0.0) / np.abs(m.y).mean()
    print(f"{wl.name}: xn off {off.mean():.1e}, moe part max_rel {mx:.3e} mean_rel {mean:.3e}")
    assert mx <= MAX_REL and mean <= MEAN_REL, (mx, mean)
    return ref


def run_plain_on(layer, xn_bits, wl):
    return device.run_once(layer, xn_bits, wl.E, wl.K)


def check_against_plain_run(wl, layer, out):
    """The plain layer on the kernel's own normalised rows: identical routing
    bits, and the block's y is x + the plain layer's output up to the two
    roundings (the MoE sum is the same fp32 value in both)."""
    plain = run_plain_on(layer, out["norm_x"], wl)
    for k in ("topk_idx", "topk_w", "pair_rank", "expert_count", "logits"):
        assert np.array_equal(plain[k], out[k]), k
    x = O.bf16_bits_to_f64(out["x"])
    yb = O.bf16_bits_to_f64(out["y"])
    yp = O.bf16_bits_to_f64(plain["y"])
    assert np.all(np.abs(yb - (x + yp)) <= bf16_half_ulp(yb) + bf16_half_ulp(yp))


def run_block(layer, inp, wl):
    out = device.run_once(layer, inp.x, wl.E, wl.K, block=True)
    out["x"] = inp.x
    return out


CASES = synth.PRENORM + [block_of(w) for w in (
    synth.Workload("t9_h4096_e256_k8_s1", T=9, H=4096, E=256, K=8, S=1, I=512),   # x in global memory
    synth.Workload("t20_h128_e8_k8_s1", T=20, H=128, E=8, K=8, S=1, I=64),        # router tiles, K = E
    synth.Workload("t33_h320_e64_k6_s1", T=33, H=320, E=64, K=6, S=1, I=128, zipf_s=1.2),
    synth.Workload("t6_h4096_e256_k8_s1_i576", T=6, H=4096, E=256, K=8, S=1, I=576),
)]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_block_parity(wl):
    print(f"case {wl.name}", flush=True)
    inp = inputs_for(wl)
    layer = device.make_layer(inp)
    out = run_block(layer, inp, wl)
    rows = None
    if wl.T > 64:
        rows = np.sort(np.random.default_rng(1).choice(wl.T, 40, replace=False))
    check_block(wl, inp, out, rows)
    check_against_plain_run(wl, layer, out)
    again = run_block(layer, inp, wl)
    assert np.array_equal(again["y"], out["y"]) and np.array_equal(again["norm_x"], out["norm_x"])
    layer.close()


@pytest.mark.parametrize("base,Ts", [(1, (6, 1, 4, 6)), (4, (384, 17, 200, 45))],
                         ids=["small", "wide"])
def test_block_and_plain_runs_alternate_on_one_handle(base, Ts):
    """Block runs of changing row counts, each followed by a plain run on the
    same handle: every block run matches the oracle (the row ready words of
    one run never pass for another's)."""
    wl = synth.PRENORM[base]
    inp = inputs_for(wl)
    layer = device.make_layer(inp, max_tokens=wl.T)
    for T in Ts:
        print(f"case {wl.name} T={T}", flush=True)
        sub = dataclasses.replace(inp, workload=wl.with_rows(T), x=inp.x[:T], attempts=inp.attempts[:T])
        out = run_block(layer, sub, sub.workload)
        rows = None if T <= 64 else np.sort(np.random.default_rng(T).choice(T, 24, replace=False))
        check_block(sub.workload, sub, out, rows)
        plain = device.run_once(layer, out["norm_x"], wl.E, wl.K)
        assert np.array_equal(plain["topk_idx"], out["topk_idx"])
    layer.close()


def test_block_run_needs_the_norm_weight_and_rejects_bad_epsilon():
    wl = synth.BY_NAME["tiny_t4_h256_e16_k2"]
    inp = synth.make_inputs(wl)
    layer = device.make_layer(inp)
    dev = torch.device("cuda", 0)
    x = device.to_device(inp.x, dev)
    y = torch.empty_like(x)
    L = binding.lib()
    s = torch.cuda.current_stream().cuda_stream
    assert L.moe_decode_run_block(layer.handle, x.data_ptr(), wl.T, y.data_ptr(), None, s) == \
        binding.MOE_ERR_INVALID_ARG
    g = torch.ones(wl.H, dtype=torch.float32, device=dev)
    for eps in (0.0, -1e-6, float("inf"), float("nan")):
        assert L.moe_decode_set_input_norm(layer.handle, g.data_ptr(), eps) == binding.MOE_ERR_INVALID_ARG
    assert L.moe_decode_set_input_norm(layer.handle, None, 1e-6) == binding.MOE_ERR_INVALID_ARG
    layer.set_input_norm(g, 1e-6)
    layer.run_block(x, y, wl.T)
    assert layer.check() == binding.MOE_OK
    layer.close()


def test_expired_waits_in_a_block_run_report_timeout_and_the_next_run_recovers():
    wl = synth.PRENORM[1]
    inp = inputs_for(wl)
    layer = device.make_layer(inp)
    dev = torch.device("cuda", 0)
    x = device.to_device(inp.x, dev)
    y = torch.empty_like(x)
    print("case expired waits, block run", flush=True)
    layer.run_block(x, y, wl.T, {"expire_waits": 1})
    assert layer.check() == binding.MOE_ERR_TIMEOUT
    out = run_block(layer, inp, wl)
    check_block(wl, inp, out)
    layer.close()
