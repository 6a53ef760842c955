"""Device plumbing: copy host inputs into torch device memory and call the layer.

torch only allocates memory and provides the stream; the layer itself runs in
the HIP library through ``binding``.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding
from .synth import Inputs


def to_device(a: np.ndarray, dev) -> torch.Tensor:
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(dev).contiguous()


def upload_weights(inp: Inputs, dev) -> dict:
    return {
        "router_w": to_device(inp.router_w, dev),
        "router_bias": None if inp.router_b is None else to_device(inp.router_b, dev),
        "w13": to_device(inp.w13, dev),
        "s13": to_device(inp.s13, dev),
        "w2": to_device(inp.w2, dev),
        "s2": to_device(inp.s2, dev),
    }


def make_layer(inp: Inputs, max_tokens: int | None = None, device: int = 0,
               deadline_us: int = 0, free_weights: bool = True, cooperative: bool = False) -> binding.MoeDecode:
    """Create a handle for the inputs' workload; the standard-layout weight
    copies are dropped after create (the handle holds its own tile layout)."""
    wl = inp.workload
    dev = torch.device("cuda", device)
    w = upload_weights(inp, dev)
    cfg = binding.make_config(max_tokens or wl.T, wl.H, wl.E, wl.K, wl.I, wl.S, deadline_us,
                              wl.weight_format, cooperative)
    layer = binding.MoeDecode(cfg, w, device)
    if wl.prenorm:
        layer.set_input_norm(to_device(inp.norm_w, dev), wl.norm_eps)
    if wl.swiglu_limit is not None:
        layer.set_swiglu_limit(wl.swiglu_limit)
    if free_weights:
        del w
        torch.cuda.empty_cache()
    return layer


def debug_buffers(T: int, E: int, K: int, dev) -> dict:
    return {
        "topk_idx": torch.full((T, K), -1, dtype=torch.int32, device=dev),
        "topk_w": torch.full((T, K), float("nan"), dtype=torch.float32, device=dev),
        "pair_rank": torch.full((T, K), -1, dtype=torch.int32, device=dev),
        "expert_count": torch.full((E,), -1, dtype=torch.int32, device=dev),
        "logits": torch.full((T, E), float("nan"), dtype=torch.float32, device=dev),
    }


def run_once(layer: binding.MoeDecode, x_bits: np.ndarray, E: int, K: int, device: int = 0,
             debug: bool = True, block: bool = False) -> dict:
    """One synchronous call (a pre-norm block call with ``block``); returns y
    (bf16 bits, uint16) and the debug copies."""
    dev = torch.device("cuda", device)
    T, H = x_bits.shape
    x = to_device(x_bits, dev)
    y = torch.full((T, H), -1, dtype=torch.int16, device=dev)
    dbg = debug_buffers(T, E, K, dev) if debug else None
    if block:
        if dbg is not None:
            dbg["norm_x"] = torch.full((T, H), -1, dtype=torch.int16, device=dev)
        layer.run_block(x, y, T, dbg)
    else:
        layer.run(x, y, T, dbg)
    st = layer.check()
    if st != binding.MOE_OK:
        raise binding.MoeDecodeError("moe_decode_check", st)
    out = {"y": y.cpu().numpy().view(np.uint16)}
    if dbg:
        for k, v in dbg.items():
            out[k] = v.cpu().numpy()
        if "norm_x" in out:
            out["norm_x"] = out["norm_x"].view(np.uint16)
    return out
