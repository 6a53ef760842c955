"""moe_decode_run_static: the layer with its whole workspace in the library's
static per-GPU array (no allocation), against moe_decode_run on the same
handle and inputs.  Both run the same kernel on the same data in the same
order, so the outputs must agree bit for bit (within the layer's bars a
fortiori); the first call is also held to the oracle."""
import json
import os

import numpy as np
import pytest
import torch

from checks import MAX_REL, MEAN_REL, output_errors
from moe_decode_layer_amd import binding, device, synth
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "attempts.json")))


def _run(layer, x_bits, E, K, static):
    dev = torch.device("cuda", 0)
    T = x_bits.shape[0]
    x = device.to_device(np.ascontiguousarray(x_bits), dev)
    y = torch.full_like(x, -1)
    dbg = device.debug_buffers(T, E, K, dev)
    (layer.run_static if static else layer.run)(x, y, T, dbg)
    assert layer.check() == binding.MOE_OK
    out = {k: v.cpu().numpy() for k, v in dbg.items()}
    out["y"] = y.cpu().numpy().view(np.uint16)
    return out


def _same(a, b, what):
    for k in ("y", "topk_idx", "topk_w", "pair_rank", "expert_count", "logits"):
        assert np.array_equal(a[k], b[k]), f"{what}: {k} differs"


def test_static_workspace_matches_the_handle_workspace():
    wa = synth.WORKLOADS[1]          # 6 rows, H 4096, 256 experts top-8 + shared, I 512
    wb = synth.WORKLOADS[0]          # 4 rows, H 256, 16 experts top-2, I 128
    print(f"case static workspace {wa.name} then {wb.name}", flush=True)
    ia = synth.make_inputs(wa, GOLDEN["attempts"][wa.name])
    ib = synth.make_inputs(wb, GOLDEN["attempts"][wb.name])
    la, lb = device.make_layer(ia), device.make_layer(ib)
    # two calls in a row on one handle, the second with fewer rows
    ref6 = _run(la, ia.x, wa.E, wa.K, static=False)
    got6 = _run(la, ia.x, wa.E, wa.K, static=True)
    _same(got6, ref6, "6 rows")
    r = O.forward(ia)
    mx, mean = output_errors(O.bf16_bits_to_f64(got6["y"]), r.y_bf16)
    assert mx <= MAX_REL and mean <= MEAN_REL, (mx, mean)
    ref3 = _run(la, ia.x[:3], wa.E, wa.K, static=False)
    got3 = _run(la, ia.x[:3], wa.E, wa.K, static=True)
    _same(got3, ref3, "3 rows after 6")
    # another handle (another shape) on the same array, then the first again
    refb = _run(lb, ib.x, wb.E, wb.K, static=False)
    gotb = _run(lb, ib.x, wb.E, wb.K, static=True)
    _same(gotb, refb, "second handle")
    again = _run(la, ia.x[:5], wa.E, wa.K, static=True)
    _same(again, _run(la, ia.x[:5], wa.E, wa.K, static=False), "first handle again, 5 rows")
    la.close()
    lb.close()


def test_static_workspace_with_mxfp4_weights():
    """The MXFP4 full-tile kernel (two row blocks per gate/up item at 6 and 4
    rows, one at 2) on the static array, against the handle workspace."""
    wl = synth.BY_NAME["verify_t6_h4096_e256_k8_s1_mxfp4"]
    print(f"case static workspace {wl.name}", flush=True)
    inp = synth.make_inputs(wl, GOLDEN["attempts"][wl.name])
    layer = device.make_layer(inp)
    for T in (6, 4, 2):
        ref = _run(layer, inp.x[:T], wl.E, wl.K, static=False)
        got = _run(layer, inp.x[:T], wl.E, wl.K, static=True)
        _same(got, ref, f"MXFP4, {T} rows")
    r = O.forward(inp)
    mx, mean = output_errors(O.bf16_bits_to_f64(_run(layer, inp.x, wl.E, wl.K, static=True)["y"]), r.y_bf16)
    assert mx <= MAX_REL and mean <= MEAN_REL, (mx, mean)
    layer.close()


def test_static_workspace_limit_timeout_and_recovery():
    wa = synth.WORKLOADS[1]
    print(f"case static workspace limit {wa.name}", flush=True)
    ia = synth.make_inputs(wa, GOLDEN["attempts"][wa.name])
    layer = device.make_layer(ia, max_tokens=64)
    dev = torch.device("cuda", 0)
    x = torch.zeros((64, wa.H), dtype=torch.int16, device=dev)
    y = torch.empty_like(x)
    # 64 rows need more than the array holds at this shape: refused up front
    st = binding.moe_decode_run_static(layer.handle, x.data_ptr(), 64, y.data_ptr(), None,
                                       torch.cuda.current_stream().cuda_stream)
    assert st == binding.MOE_ERR_UNSUPPORTED
    # a failed wait reports through check, and the next call is clean
    xs = device.to_device(ia.x, dev)
    ys = torch.empty_like(xs)
    layer.run_static(xs, ys, wa.T, {"expire_waits": 1})
    assert layer.check() == binding.MOE_ERR_TIMEOUT
    assert layer.check() == binding.MOE_OK
    got = _run(layer, ia.x, wa.E, wa.K, static=True)
    _same(got, _run(layer, ia.x, wa.E, wa.K, static=False), "after a timeout")
    layer.close()
