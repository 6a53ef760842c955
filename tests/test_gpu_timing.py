"""moe_decode_set_launch_events: runs launched with the kernel's own start and
stop events.  The outputs are those of a run without events, bit for bit; the
kernel events fall inside event records queued around the call; clearing the
events restores plain launches; a cooperative handle, and a stream that is
capturing a graph, refuse timed runs."""
import json
import os

import numpy as np
import pytest
import torch

from moe_decode_layer_amd import binding, device, synth

pytestmark = pytest.mark.gpu

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "attempts.json")))


def _events(n):
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    s = torch.cuda.current_stream()
    for e in ev:
        e.record(s)          # the events exist once recorded
    torch.cuda.synchronize()
    return ev


def test_launch_events_time_the_kernel_itself():
    wl = synth.WORKLOADS[1]          # 6 rows, H 4096, 256 experts top-8 + shared, I 512
    print(f"case launch events {wl.name}", flush=True)
    inp = synth.make_inputs(wl, GOLDEN["attempts"][wl.name])
    layer = device.make_layer(inp)
    dev = torch.device("cuda", 0)
    x = device.to_device(inp.x, dev)
    y0 = torch.full_like(x, -1)
    layer.run(x, y0)
    torch.cuda.synchronize()
    assert layer.check() == binding.MOE_OK
    k0, k1, o0, o1 = _events(4)
    s = torch.cuda.current_stream()
    kernel_ms, outer_ms = [], []
    for r in range(3):
        y1 = torch.full_like(x, -1)
        layer.set_launch_events(k0, k1)
        o0.record(s)
        layer.run(x, y1)
        o1.record(s)
        torch.cuda.synchronize()
        assert layer.check() == binding.MOE_OK
        assert torch.equal(y1.view(torch.int16), y0.view(torch.int16)), f"timed run {r} differs"
        kernel_ms.append(k0.elapsed_time(k1))
        outer_ms.append(o0.elapsed_time(o1))
    print("kernel ms", np.round(kernel_ms, 4), "outer ms", np.round(outer_ms, 4))
    for k, o in zip(kernel_ms, outer_ms):
        assert 0.0 < k <= o
    # cleared: plain launches again (the old events are no longer touched)
    layer.set_launch_events(None, None)
    before = k0.elapsed_time(k1)
    y2 = torch.full_like(x, -1)
    layer.run(x, y2)
    torch.cuda.synchronize()
    assert layer.check() == binding.MOE_OK
    assert torch.equal(y2.view(torch.int16), y0.view(torch.int16))
    assert k0.elapsed_time(k1) == before
    layer.close()


def test_cooperative_handle_refuses_timed_runs():
    wl = synth.WORKLOADS[0]          # tiny
    print(f"case cooperative + launch events {wl.name}", flush=True)
    inp = synth.make_inputs(wl, GOLDEN["attempts"][wl.name])
    layer = device.make_layer(inp, cooperative=True)
    dev = torch.device("cuda", 0)
    x = device.to_device(inp.x, dev)
    y = torch.empty_like(x)
    k0, k1 = _events(2)
    layer.set_launch_events(k0, k1)
    with pytest.raises(binding.MoeDecodeError) as e:
        layer.run(x, y)
    assert e.value.status == binding.MOE_ERR_UNSUPPORTED
    layer.set_launch_events(None, None)
    layer.run(x, y)
    torch.cuda.synchronize()
    assert layer.check() == binding.MOE_OK
    layer.close()


def test_launch_events_refused_under_graph_capture():
    wl = synth.WORKLOADS[0]          # tiny
    print(f"case launch events under capture {wl.name}", flush=True)
    inp = synth.make_inputs(wl, GOLDEN["attempts"][wl.name])
    layer = device.make_layer(inp)
    dev = torch.device("cuda", 0)
    x = device.to_device(inp.x, dev)
    y = torch.empty_like(x)
    layer.run(x, y)                  # eager first (occupancy query outside the capture)
    torch.cuda.synchronize()
    k0, k1 = _events(2)
    before = k0.elapsed_time(k1)     # the two records of _events
    layer.set_launch_events(k0, k1)
    g = torch.cuda.CUDAGraph()
    status = None
    with torch.cuda.graph(g):
        y.zero_()                    # the graph holds this one node
        try:
            layer.run(x, y)
        except binding.MoeDecodeError as e:
            status = e.status
    assert status == binding.MOE_ERR_UNSUPPORTED
    # eager runs with the same events still time the kernel
    y1 = torch.full_like(x, -1)
    layer.run(x, y1)
    torch.cuda.synchronize()
    assert layer.check() == binding.MOE_OK
    assert k0.elapsed_time(k1) > 0.0 and k0.elapsed_time(k1) != before
    layer.set_launch_events(None, None)
    layer.close()
