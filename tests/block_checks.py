"""Checks of pre-norm block runs against the oracle, shared by the block and
clipped-SwiGLU GPU tests.

The block output y = bf16(x + moe(xn)) is held to the layer's bars in two
steps: the plain layer run on the kernel's own normalised rows must meet the
max and mean bars against the oracle on those rows, and the block's y must
equal x + that plain output up to the two roundings.
"""
import dataclasses

import numpy as np

from checks import MAX_REL, MEAN_REL, check_placement, output_errors
from moe_decode_layer_amd import device
from oracle import moe_oracle as O


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
    # a coarse bound on y itself: its own rounding plus the layer's max bar;
    # the strict bars are applied in check_against_plain_run
    y = O.bf16_bits_to_f64(out["y"])[ref.moe.rows]
    assert np.all(np.abs(y - ref.y) <= bf16_half_ulp(y) + MAX_REL * np.abs(m.y).max())
    print(f"{wl.name}: xn off {off.mean():.1e}", flush=True)
    return ref


def check_against_plain_run(wl, inp, layer, out):
    """The plain layer run on the kernel's own normalised rows: its y meets
    the layer's bars (max and mean) against the oracle on those same rows;
    its routing bits equal the block run's; and the block's y is x + the
    plain layer's output up to the two roundings (the MoE sum is the same
    fp32 value in both)."""
    plain = device.run_once(layer, out["norm_x"], wl.E, wl.K)
    for k in ("topk_idx", "topk_w", "pair_rank", "expert_count", "logits"):
        assert np.array_equal(plain[k], out[k]), k
    ref = O.forward(dataclasses.replace(inp, x=out["norm_x"]))
    assert np.array_equal(plain["topk_idx"], ref.idx)
    yp = O.bf16_bits_to_f64(plain["y"])
    mx, mean = output_errors(yp, ref.y_bf16)
    print(f"{wl.name}: moe part (plain run on the kernel's xn) max_rel {mx:.3e} mean_rel {mean:.3e}",
          flush=True)
    assert mx <= MAX_REL and mean <= MEAN_REL, (mx, mean)
    x = O.bf16_bits_to_f64(out["x"])
    yb = O.bf16_bits_to_f64(out["y"])
    assert np.all(np.abs(yb - (x + yp)) <= bf16_half_ulp(yb) + bf16_half_ulp(yp))


def run_block(layer, inp, wl):
    out = device.run_once(layer, inp.x, wl.E, wl.K, block=True)
    out["x"] = inp.x
    return out


def rolled(inp, shift, T=None):
    """The inputs with their rows rotated by ``shift`` (and cut to T rows):
    every row keeps its own routing margins, but each run on a handle sees
    different rows in each position, so a stale normalised row left by an
    earlier run can never pass for the current one."""
    T = inp.workload.T if T is None else T
    x = np.ascontiguousarray(np.roll(inp.x, shift, axis=0)[:T])
    att = np.roll(inp.attempts, shift)[:T]
    return dataclasses.replace(inp, workload=inp.workload.with_rows(T) if T != inp.workload.T else inp.workload,
                               x=x, attempts=att)
