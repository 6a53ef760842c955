"""ctypes binding of the C ABI in include/moe_decode.h (argument marshalling only).

The functions keep the C names.  Tensors are torch tensors on the handle's
device; only their data pointers cross the boundary.  Every step of the layer
runs in the HIP library; if it has not been built, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_moe_decode.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_HIP = 3
MOE_ERR_OUT_OF_MEMORY = 4
MOE_ERR_TIMEOUT = 5

# Expert weight formats (config flags, bits 0-1) and, per format, the bytes
# of codes per 2 elements and the scale dtype.
MOE_WEIGHTS_FP8 = 0
MOE_WEIGHTS_MXFP8 = 1
MOE_WEIGHTS_MXFP4 = 2
WEIGHT_FORMATS = {"fp8": MOE_WEIGHTS_FP8, "mxfp8": MOE_WEIGHTS_MXFP8, "mxfp4": MOE_WEIGHTS_MXFP4}
MOE_FLAG_COOPERATIVE = 4

# Functions declared in include/moe_decode.h, in declaration order.
EXPORTS = (
    "moe_decode_abi_version",
    "moe_decode_supported",
    "moe_decode_create",
    "moe_decode_run",
    "moe_decode_run_static",
    "moe_decode_set_input_norm",
    "moe_decode_run_block",
    "moe_decode_set_swiglu_limit",
    "moe_decode_set_launch_events",
    "moe_decode_check",
    "moe_decode_destroy",
    "moe_decode_status_string",
)



class moe_decode_config(ctypes.Structure):
    _fields_ = [
        ("max_tokens", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("intermediate", ctypes.c_int32),
        ("num_shared", ctypes.c_int32),
        ("deadline_us", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
    ]


class moe_decode_weights(ctypes.Structure):
    _fields_ = [
        ("router_w", ctypes.c_void_p),
        ("router_bias", ctypes.c_void_p),
        ("w13", ctypes.c_void_p),
        ("s13", ctypes.c_void_p),
        ("w2", ctypes.c_void_p),
        ("s2", ctypes.c_void_p),
    ]


class moe_decode_debug(ctypes.Structure):
    _fields_ = [
        ("topk_idx", ctypes.c_void_p),
        ("topk_w", ctypes.c_void_p),
        ("pair_rank", ctypes.c_void_p),
        ("expert_count", ctypes.c_void_p),
        ("logits", ctypes.c_void_p),
        ("trace", ctypes.c_void_p),
        ("trace_blocks", ctypes.c_int32),
        ("trace_cap", ctypes.c_int32),
        ("expire_waits", ctypes.c_int32),
        ("norm_x", ctypes.c_void_p),
    ]


class MoeDecodeError(RuntimeError):
    def __init__(self, where: str, status: int):
        super().__init__(f"{where}: {moe_decode_status_string(status)} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: run __graft_entry__.build() to compile the HIP library")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.moe_decode_abi_version.restype = ctypes.c_int32
        L.moe_decode_abi_version.argtypes = []
        L.moe_decode_supported.restype = ctypes.c_int32
        L.moe_decode_supported.argtypes = [ctypes.POINTER(moe_decode_config), ctypes.c_int32]
        L.moe_decode_create.restype = ctypes.c_int32
        L.moe_decode_create.argtypes = [ctypes.POINTER(moe_decode_config),
                                        ctypes.POINTER(moe_decode_weights), ctypes.c_int32,
                                        ctypes.POINTER(P)]
        L.moe_decode_run.restype = ctypes.c_int32
        L.moe_decode_run.argtypes = [P, P, ctypes.c_int32, P, ctypes.POINTER(moe_decode_debug), P]
        L.moe_decode_run_static.restype = ctypes.c_int32
        L.moe_decode_run_static.argtypes = [P, P, ctypes.c_int32, P, ctypes.POINTER(moe_decode_debug), P]
        L.moe_decode_set_input_norm.restype = ctypes.c_int32
        L.moe_decode_set_input_norm.argtypes = [P, P, ctypes.c_float]
        L.moe_decode_run_block.restype = ctypes.c_int32
        L.moe_decode_run_block.argtypes = [P, P, ctypes.c_int32, P, ctypes.POINTER(moe_decode_debug), P]
        L.moe_decode_set_swiglu_limit.restype = ctypes.c_int32
        L.moe_decode_set_swiglu_limit.argtypes = [P, ctypes.c_float]
        L.moe_decode_set_launch_events.restype = ctypes.c_int32
        L.moe_decode_set_launch_events.argtypes = [P, P, P]
        L.moe_decode_check.restype = ctypes.c_int32
        L.moe_decode_check.argtypes = [P]
        L.moe_decode_destroy.restype = None
        L.moe_decode_destroy.argtypes = [P]
        L.moe_decode_status_string.restype = ctypes.c_char_p
        L.moe_decode_status_string.argtypes = [ctypes.c_int32]
        _lib = L
    return _lib


# ---- thin wrappers with the C names ---------------------------------------
def moe_decode_abi_version() -> int:
    return lib().moe_decode_abi_version()


def moe_decode_status_string(status: int) -> str:
    return lib().moe_decode_status_string(status).decode()


def moe_decode_supported(cfg: moe_decode_config, T: int) -> int:
    return lib().moe_decode_supported(ctypes.byref(cfg), T)


def moe_decode_create(cfg: moe_decode_config, w: moe_decode_weights, device: int):
    h = ctypes.c_void_p()
    st = lib().moe_decode_create(ctypes.byref(cfg), ctypes.byref(w), device, ctypes.byref(h))
    return st, h


def moe_decode_run(h, x_ptr: int, T: int, y_ptr: int, dbg: moe_decode_debug | None,
                   stream: int) -> int:
    return lib().moe_decode_run(h, x_ptr, T, y_ptr, ctypes.byref(dbg) if dbg is not None else None,
                                stream)


def moe_decode_run_static(h, x_ptr: int, T: int, y_ptr: int, dbg: moe_decode_debug | None,
                          stream: int) -> int:
    return lib().moe_decode_run_static(h, x_ptr, T, y_ptr, ctypes.byref(dbg) if dbg is not None else None,
                                       stream)


def moe_decode_set_input_norm(h, norm_w_ptr: int, eps: float) -> int:
    return lib().moe_decode_set_input_norm(h, norm_w_ptr, eps)


def moe_decode_run_block(h, x_ptr: int, T: int, y_ptr: int, dbg: moe_decode_debug | None,
                         stream: int) -> int:
    return lib().moe_decode_run_block(h, x_ptr, T, y_ptr,
                                      ctypes.byref(dbg) if dbg is not None else None, stream)


def moe_decode_set_swiglu_limit(h, limit: float) -> int:
    return lib().moe_decode_set_swiglu_limit(h, limit)


def moe_decode_set_launch_events(h, start_event: int | None, stop_event: int | None) -> int:
    return lib().moe_decode_set_launch_events(h, start_event, stop_event)


def moe_decode_check(h) -> int:
    return lib().moe_decode_check(h)


def moe_decode_destroy(h) -> None:
    lib().moe_decode_destroy(h)


# ---- convenience layer over torch tensors ---------------------------------
def make_config(T_max, H, E, K, I, S, deadline_us=0, weight_format: str = "fp8",
                cooperative: bool = False) -> moe_decode_config:
    flags = WEIGHT_FORMATS[weight_format] | (MOE_FLAG_COOPERATIVE if cooperative else 0)
    return moe_decode_config(T_max, H, E, K, I, S, deadline_us, flags)


def weight_layout(cfg: moe_decode_config, bias: bool = False) -> dict:
    """Element type name and element count of each weight array the header
    gives for the config's format: codes one byte per element (MXFP4: two
    elements per byte), scales fp32 (FP8) or E8M0 bytes (MX), one per 32 K."""
    fmt = cfg.flags & 3
    E, S, H, I = cfg.num_experts, cfg.num_shared, cfg.hidden, cfg.intermediate
    codes = (lambda n: n // 2) if fmt == MOE_WEIGHTS_MXFP4 else (lambda n: n)
    scale = "float32" if fmt == MOE_WEIGHTS_FP8 else "uint8"
    out = {"router_w": ("float32", E * H), "w13": ("uint8", (E + S) * 2 * I * codes(H)),
           "s13": (scale, (E + S) * 2 * I * (H // 32)), "w2": ("uint8", (E + S) * H * codes(I)),
           "s2": (scale, (E + S) * H * (I // 32))}
    if bias:
        out["router_bias"] = ("float32", E)
    return out


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


class MoeDecode:
    """One handle: weights re-laid out on the device, workspace for max_tokens rows.

    ``weights`` maps router_w, router_bias (or None), w13, s13, w2, s2 to
    contiguous torch tensors on ``device`` in the layouts of the header.
    """

    def __init__(self, cfg: moe_decode_config, weights: dict, device: int = 0):
        self._check_weights(cfg, weights, device)
        w = moe_decode_weights(_ptr(weights["router_w"]), _ptr(weights.get("router_bias")),
                               _ptr(weights["w13"]), _ptr(weights["s13"]),
                               _ptr(weights["w2"]), _ptr(weights["s2"]))
        st, h = moe_decode_create(cfg, w, device)
        if st != MOE_OK:
            raise MoeDecodeError("moe_decode_create", st)
        self.cfg = cfg
        self.device = device
        self.handle = h

    @staticmethod
    def _check_weights(cfg: moe_decode_config, weights: dict, device: int) -> None:
        """Every weight tensor contiguous, on the device, with the element type
        and count of weight_layout (create reads them whole: a short tensor
        would be read past its end)."""
        for name, (dtype, n) in weight_layout(cfg, weights.get("router_bias") is not None).items():
            t = weights[name]
            if not (t.is_cuda and t.device.index == device and t.is_contiguous()):
                raise ValueError(f"{name}: must be a contiguous tensor on cuda:{device}")
            if str(t.dtype).removeprefix("torch.") != dtype or t.numel() != n:
                raise ValueError(f"{name}: expected {n} elements of {dtype}, got {t.numel()} of {t.dtype}")

    def _check_rows(self, name: str, t, T: int) -> None:
        """x and y: 2-byte elements, contiguous, on the handle's device, at
        least T rows of H.  A short or misplaced buffer would make the kernel
        read or write past it, so the call is refused here instead."""
        if t is None:
            raise ValueError(f"{name} is required")
        if t.element_size() != 2 or not t.is_cuda or t.device.index != self.device:
            raise ValueError(f"{name}: need a 2-byte (bf16) tensor on cuda:{self.device}, "
                             f"got {t.dtype} on {t.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.numel() < T * self.cfg.hidden:
            raise ValueError(f"{name} holds {t.numel()} elements, fewer than T*H = "
                             f"{T} * {self.cfg.hidden}")

    def _check_debug(self, debug: dict | None, T: int) -> None:
        """Each debug buffer is contiguous, on the device, with 4-byte (or,
        for norm_x, 2-byte; trace: 8-byte) elements, at least as large as
        its field needs."""
        if not debug:
            return
        K, E, H = self.cfg.top_k, self.cfg.num_experts, self.cfg.hidden
        need = {"topk_idx": (T * K, 4), "topk_w": (T * K, 4), "pair_rank": (T * K, 4),
                "expert_count": (E, 4), "logits": (T * E, 4), "norm_x": (T * H, 2)}
        for name, (n, size) in need.items():
            t = debug.get(name)
            if t is None:
                continue
            if (not t.is_cuda or t.device.index != self.device or not t.is_contiguous()
                    or t.element_size() != size or t.numel() < n):
                raise ValueError(f"debug buffer {name}: need >= {n} contiguous {size}-byte "
                                 f"elements on cuda:{self.device}")
        tr = debug.get("trace")
        if tr is not None:
            if (not tr.is_cuda or tr.device.index != self.device or not tr.is_contiguous()
                    or tr.element_size() != 8 or tr.dim() != 3 or tr.shape[1] < 2 or tr.shape[2] != 4):
                raise ValueError("debug trace: need a contiguous int64 [blocks][1 + cap][4] tensor")

    @staticmethod
    def _debug(debug: dict | None):
        if not debug:
            return None
        tr = debug.get("trace")
        return moe_decode_debug(_ptr(debug.get("topk_idx")), _ptr(debug.get("topk_w")),
                                _ptr(debug.get("pair_rank")), _ptr(debug.get("expert_count")),
                                _ptr(debug.get("logits")), _ptr(tr),
                                0 if tr is None else tr.shape[0],
                                0 if tr is None else tr.shape[1] - 1,
                                int(debug.get("expire_waits", 0)), _ptr(debug.get("norm_x")))

    def run(self, x, y, T: int | None = None, debug: dict | None = None, stream=None) -> None:
        """Enqueue one layer call: x [T][H] bf16 -> y [T][H] bf16 (torch tensors)."""
        import torch
        if T is None:
            T = x.shape[0]
        if T > 0:
            self._check_rows("x", x, T)
            self._check_rows("y", y, T)
            self._check_debug(debug, T)
        s = stream if stream is not None else torch.cuda.current_stream()
        st = moe_decode_run(self.handle, x.data_ptr(), T, y.data_ptr(), self._debug(debug),
                            s.cuda_stream)
        if st != MOE_OK:
            raise MoeDecodeError("moe_decode_run", st)

    def run_static(self, x, y, T: int | None = None, debug: dict | None = None, stream=None) -> None:
        """Like run, with the workspace in the library's static array (no allocation)."""
        import torch
        if T is None:
            T = x.shape[0]
        if T > 0:
            self._check_rows("x", x, T)
            self._check_rows("y", y, T)
            self._check_debug(debug, T)
        s = stream if stream is not None else torch.cuda.current_stream()
        st = moe_decode_run_static(self.handle, x.data_ptr(), T, y.data_ptr(), self._debug(debug),
                                   s.cuda_stream)
        if st != MOE_OK:
            raise MoeDecodeError("moe_decode_run_static", st)

    def set_input_norm(self, norm_w, eps: float) -> None:
        """RMSNorm weight [H] fp32 (torch tensor on the device) and epsilon of block runs."""
        assert norm_w.is_cuda and norm_w.is_contiguous()
        st = moe_decode_set_input_norm(self.handle, norm_w.data_ptr(), eps)
        if st != MOE_OK:
            raise MoeDecodeError("moe_decode_set_input_norm", st)

    def set_swiglu_limit(self, limit: float) -> None:
        """Clipped SwiGLU limit of later runs (+inf: no clipping)."""
        st = moe_decode_set_swiglu_limit(self.handle, limit)
        if st != MOE_OK:
            raise MoeDecodeError("moe_decode_set_swiglu_limit", st)

    def set_launch_events(self, start=None, stop=None) -> None:
        """Kernel start and stop events for later runs (torch.cuda.Event with
        timing, already recorded once so that they exist), or None, None to
        turn timing off."""
        def raw(e):
            if e is None:
                return None
            if not e.cuda_event:
                raise ValueError("the event has not been created yet: record it once first")
            return e.cuda_event
        st = moe_decode_set_launch_events(self.handle, raw(start), raw(stop))
        if st != MOE_OK:
            raise MoeDecodeError("moe_decode_set_launch_events", st)

    def run_block(self, x, y, T: int | None = None, debug: dict | None = None, stream=None) -> None:
        """Enqueue one pre-norm block call: y = x + layer(RMSNorm(x)), [T][H] bf16."""
        import torch
        if T is None:
            T = x.shape[0]
        if T > 0:
            self._check_rows("x", x, T)
            self._check_rows("y", y, T)
            self._check_debug(debug, T)
        s = stream if stream is not None else torch.cuda.current_stream()
        st = moe_decode_run_block(self.handle, x.data_ptr(), T, y.data_ptr(), self._debug(debug),
                                  s.cuda_stream)
        if st != MOE_OK:
            raise MoeDecodeError("moe_decode_run_block", st)

    def check(self) -> int:
        return moe_decode_check(self.handle)

    def close(self) -> None:
        if self.handle:
            moe_decode_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
