"""The C-ABI library loads, exports every function include/moe_decode.h declares,
and its host-side argument checks (Guard) answer without touching a GPU."""
import ctypes
import os
import re

import pytest

from moe_decode_layer_amd import binding

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADERS = ("moe_decode.h",)


def declared_functions():
    names = []
    for h in HEADERS:
        text = open(os.path.join(INCLUDE, h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(moe_decode_\w+)\s*\(", text, flags=re.M)
    return names


def test_every_header_is_listed():
    assert sorted(f for f in os.listdir(INCLUDE) if f.endswith(".h")) == sorted(HEADERS)


def test_header_declarations_match_binding():
    assert tuple(declared_functions()) == binding.EXPORTS


def test_library_exports_every_declared_symbol():
    L = binding.lib()
    for name in declared_functions():
        assert isinstance(getattr(L, name), ctypes._CFuncPtr), name


def test_abi_version_and_status_strings():
    assert binding.moe_decode_abi_version() == 5
    # the check build() runs after compiling: libraries agree with their sources
    import sys
    sys.path.insert(0, os.path.dirname(INCLUDE))
    import __graft_entry__
    __graft_entry__.check_abi()
    for st in range(6):
        assert binding.moe_decode_status_string(st) != "unknown status"
    assert binding.moe_decode_status_string(99) == "unknown status"


def cfg(**kw):
    base = dict(T_max=384, H=4096, E=256, K=8, I=512, S=1, fmt="fp8")
    base.update(kw)
    return binding.make_config(base["T_max"], base["H"], base["E"], base["K"], base["I"], base["S"],
                               weight_format=base["fmt"])


def raw_flags(flags, **kw):
    c = cfg(**kw)
    c.flags = flags
    return c


@pytest.mark.parametrize("kw,T,want", [
    ({}, 6, binding.MOE_OK),
    ({}, 384, binding.MOE_OK),
    ({}, 0, binding.MOE_OK),
    ({}, 385, binding.MOE_ERR_UNSUPPORTED),
    ({}, -1, binding.MOE_ERR_INVALID_ARG),
    ({"H": 4000}, 6, binding.MOE_ERR_UNSUPPORTED),
    ({"I": 576}, 6, binding.MOE_OK),
    ({"I": 96}, 6, binding.MOE_OK),                  # multiple of 32: padded to 128
    ({"I": 288}, 6, binding.MOE_OK),                 # the pages' TP8 width, padded to 320
    ({"I": 80}, 6, binding.MOE_ERR_UNSUPPORTED),
    ({"H": 4064}, 6, binding.MOE_ERR_UNSUPPORTED),   # H must be a multiple of 64
    ({"K": 17, "E": 32}, 6, binding.MOE_ERR_UNSUPPORTED),
    ({"K": 9, "E": 8}, 6, binding.MOE_ERR_UNSUPPORTED),
    ({"E": 257}, 6, binding.MOE_ERR_UNSUPPORTED),
    ({"S": 2}, 6, binding.MOE_ERR_UNSUPPORTED),
    ({"T_max": 513}, 6, binding.MOE_ERR_UNSUPPORTED),
    ({"T_max": 0}, 0, binding.MOE_ERR_INVALID_ARG),
    ({"E": 0}, 1, binding.MOE_ERR_INVALID_ARG),
    # the MX formats take the same shapes (64-K tiles, I padded to 64)
    ({"fmt": "mxfp4"}, 6, binding.MOE_OK),
    ({"fmt": "mxfp4"}, 384, binding.MOE_OK),
    ({"fmt": "mxfp4", "I": 288}, 6, binding.MOE_OK),
    ({"fmt": "mxfp8", "I": 576}, 6, binding.MOE_OK),
    ({"fmt": "mxfp4", "H": 4064}, 6, binding.MOE_ERR_UNSUPPORTED),
    ({"fmt": "mxfp8", "I": 80}, 6, binding.MOE_ERR_UNSUPPORTED),
])
def test_guard(kw, T, want):
    assert binding.moe_decode_supported(cfg(**kw), T) == want


@pytest.mark.parametrize("flags,want", [
    (0, binding.MOE_OK), (1, binding.MOE_OK), (2, binding.MOE_OK),
    (3, binding.MOE_ERR_INVALID_ARG),            # no fourth format
    (4, binding.MOE_OK), (6, binding.MOE_OK),    # cooperative launch, with any format
    (7, binding.MOE_ERR_INVALID_ARG),
    (8, binding.MOE_ERR_INVALID_ARG),            # reserved bits
    (0x80000001, binding.MOE_ERR_INVALID_ARG),
])
def test_guard_flags(flags, want):
    assert binding.moe_decode_supported(raw_flags(flags), 6) == want


@pytest.mark.parametrize("name", ["tiny_t4_h256_e16_k2", "tiny_t4_h256_e16_k2_mxfp4",
                                  "tiny_t4_h256_e16_k2_mxfp8"])
def test_weight_layout_matches_the_generator(name):
    """The arrays the binding hands to create (checked against weight_layout)
    are exactly what the input generator writes for each weight format."""
    from moe_decode_layer_amd import synth
    wl = synth.BY_NAME[name]
    c = binding.make_config(wl.T, wl.H, wl.E, wl.K, wl.I, wl.S, weight_format=wl.weight_format)
    want = binding.weight_layout(c)
    got = dict(zip(("w13", "s13", "w2", "s2"), synth.expert_weights(wl)))
    got["router_w"] = synth.router_weights(wl)
    for key, a in got.items():
        assert (str(a.dtype), a.size) == want[key], key


def test_null_arguments_are_rejected_before_any_device_call():
    L = binding.lib()
    assert L.moe_decode_supported(None, 1) == binding.MOE_ERR_INVALID_ARG
    h = ctypes.c_void_p()
    w = binding.moe_decode_weights()
    assert L.moe_decode_create(None, ctypes.byref(w), 0, ctypes.byref(h)) == binding.MOE_ERR_INVALID_ARG
    c = cfg()
    assert L.moe_decode_create(ctypes.byref(c), None, 0, ctypes.byref(h)) == binding.MOE_ERR_INVALID_ARG
    assert L.moe_decode_create(ctypes.byref(c), ctypes.byref(w), 0, ctypes.byref(h)) == \
        binding.MOE_ERR_INVALID_ARG          # NULL weight pointers
    assert L.moe_decode_create(ctypes.byref(c), ctypes.byref(w), 0, None) == binding.MOE_ERR_INVALID_ARG
    bad = cfg(H=100)
    assert L.moe_decode_create(ctypes.byref(bad), ctypes.byref(w), 0, ctypes.byref(h)) == \
        binding.MOE_ERR_UNSUPPORTED
    assert L.moe_decode_run(None, None, 1, None, None, None) == binding.MOE_ERR_INVALID_ARG
    assert L.moe_decode_run_block(None, None, 1, None, None, None) == binding.MOE_ERR_INVALID_ARG
    assert L.moe_decode_set_input_norm(None, None, 1e-6) == binding.MOE_ERR_INVALID_ARG
    assert L.moe_decode_set_swiglu_limit(None, 1.0) == binding.MOE_ERR_INVALID_ARG
    assert L.moe_decode_check(None) == binding.MOE_ERR_INVALID_ARG
    L.moe_decode_destroy(None)


def test_debug_struct_layout_matches_the_header():
    # the pointer appended for block runs sits after the three int32 fields
    assert binding.moe_decode_debug.norm_x.offset == 6 * 8 + 3 * 4 + 4
    assert ctypes.sizeof(binding.moe_decode_debug) == 6 * 8 + 3 * 4 + 4 + 8


def test_launch_events_guard():
    """The timing hook refuses a NULL handle and a half-set pair, without a GPU."""
    assert binding.moe_decode_set_launch_events(None, None, None) == binding.MOE_ERR_INVALID_ARG
    assert binding.moe_decode_set_launch_events(None, 0x1000, None) == binding.MOE_ERR_INVALID_ARG
