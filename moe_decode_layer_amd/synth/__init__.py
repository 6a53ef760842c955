"""Seeded synthetic inputs for the MoE decode layer.

The five workloads below stand in for the serving traces the pages measure
on (agent-trace replay with speculative verification; random 4K/1K and 8K/1K
requests).  Neither traces nor trained weights exist here, so every tensor
is drawn from a counter-based generator (``synth.c``) with the shapes, dtypes
and value distributions each workload names.

This module holds no arithmetic of the layer itself.  Rows of ``x`` are
drawn per (row, attempt): a caller that needs routing margins picks the
attempt of each row; the generator never looks at routing.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_synth.so")

# Stream ids of the tensors (the ``tensor`` coordinate of the generator).
TENSOR_X = 1
TENSOR_ROUTER = 2
TENSOR_W13 = 3
TENSOR_W2 = 4
TENSOR_NORM = 5


@dataclasses.dataclass(frozen=True)
class Workload:
    """One layer shape plus its value distributions.

    T rows, H hidden, E routed experts, K experts per row, S shared experts
    (0 or 1), I expert intermediate width.  ``zipf_s`` adds a Zipf(s)
    per-expert logit offset (skewed routing); None means no bias.
    """

    name: str
    T: int
    H: int
    E: int
    K: int
    S: int
    I: int
    zipf_s: float | None = None
    seed: int = 0
    x_std: float = 1.0
    expert_std: float = 0.02
    # pre-norm block: x is the residual stream, normalised (RMSNorm, weight
    # from ``norm_weight``) before the layer and added back to its output
    prenorm: bool = False
    norm_eps: float = 1e-6
    # clipped SwiGLU limit (None: no clipping)
    swiglu_limit: float | None = None
    # expert weight format: "fp8" (e4m3fn, fp32 group-32 scales), "mxfp8"
    # (e4m3fn, E8M0 group-32 scales) or "mxfp4" (E2M1, E8M0 group-32 scales)
    weight_format: str = "fp8"

    @property
    def router_std(self) -> float:
        # N(0, 1/H) read as variance 1/H, so logits come out near N(0, 1).
        return math.sqrt(1.0 / self.H)

    @property
    def n_slots(self) -> int:
        return self.E + self.S

    def expert_bytes(self) -> int:
        """Weights plus group scales of one expert (gate/up + down): FP8
        bytes and fp32 scales, MXFP8 bytes and E8M0 scales, or MXFP4 half
        bytes and E8M0 scales."""
        H, I = self.H, self.I
        elem = {"fp8": 1.0, "mxfp8": 1.0, "mxfp4": 0.5}[self.weight_format]
        scale = 4 if self.weight_format == "fp8" else 1
        return int(3 * I * H * elem) + 3 * I * (H // 32) * scale

    def with_rows(self, T: int) -> "Workload":
        return dataclasses.replace(self, T=T, name=f"{self.name}@T{T}")


# The five workloads: a tiny case the oracle finishes instantly, the
# 6-row speculative verify step (one of four tensor-parallel shares:
# intermediate 512 per GPU), plain 1-row decode, a Zipf-skewed 64-row batch
# and a 384-row verify batch (64 requests x 6 rows).
WORKLOADS = [
    Workload("tiny_t4_h256_e16_k2", T=4, H=256, E=16, K=2, S=0, I=128),
    Workload("verify_t6_h4096_e256_k8_s1", T=6, H=4096, E=256, K=8, S=1, I=512),
    Workload("decode_t1_h4096_e256_k8_s1", T=1, H=4096, E=256, K=8, S=1, I=512),
    Workload("zipf_t64_h4096_e256_k8_s1", T=64, H=4096, E=256, K=8, S=1, I=512, zipf_s=1.2),
    Workload("verify_t384_h4096_e256_k8_s1", T=384, H=4096, E=256, K=8, S=1, I=512),
]

# The same shapes as pre-norm blocks (input RMSNorm + residual add fused
# around the layer).
PRENORM = [dataclasses.replace(w, name=w.name + "_prenorm", prenorm=True) for w in WORKLOADS]

# The workloads with MX expert weights (the pages' MoE formats: MXFP4 and
# MXFP8 with E8M0 group-32 scales): 6 rows, 1 row, tiny, 64 Zipf rows and
# 384 rows.
MX = [dataclasses.replace(w, name=f"{w.name}_{fmt}", weight_format=fmt)
      for fmt in ("mxfp4", "mxfp8") for w in (WORKLOADS[1], WORKLOADS[2], WORKLOADS[0], WORKLOADS[3], WORKLOADS[4])]

# The pages' per-GPU intermediate width 576 (run natively) at 6, 64 and 384
# rows, and 384 rows at 640 (576 padded to whole 128-K tiles, as the pages'
# own kernels run it), for timing the two against each other.
WIDTHS = [dataclasses.replace(w, name=f"{w.name}_i{I}", I=I) for w, I in
          ((WORKLOADS[1], 576), (WORKLOADS[3], 576), (WORKLOADS[4], 576), (WORKLOADS[4], 640))]

BY_NAME = {w.name: w for w in WORKLOADS + PRENORM + MX + WIDTHS}

_lib = None


def lib() -> ctypes.CDLL:
    """The compiled generator; fails loudly when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: run __graft_entry__.build() to compile the generator")
        L = ctypes.CDLL(LIB_PATH)
        u64, u32, i32, i64, f64, vp = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int32,
                                       ctypes.c_int64, ctypes.c_double, ctypes.c_void_p)
        L.synth_abi.restype = ctypes.c_int
        L.synth_max_threads.restype = ctypes.c_int
        L.synth_set_threads.argtypes = [ctypes.c_int]
        L.synth_bf16_encode.argtypes = [f64]
        L.synth_bf16_encode.restype = ctypes.c_uint16
        L.synth_e4m3fn_encode.argtypes = [f64]
        L.synth_e4m3fn_encode.restype = ctypes.c_uint8
        L.synth_normal_f64.argtypes = [u64, u32, u32, u32, i64, vp]
        L.synth_u64.argtypes = [u64, u32, u32, u32, i64, vp]
        L.synth_x_bf16.argtypes = [u64, u32, i32, i32, f64, vp, vp]
        L.synth_f32.argtypes = [u64, u32, u32, i32, i32, f64, vp]
        L.synth_fp8_g32.argtypes = [u64, u32, u32, i32, i32, f64, vp, vp]
        L.synth_e2m1_encode.argtypes = [f64]
        L.synth_e2m1_encode.restype = ctypes.c_uint8
        L.synth_mx_g32.argtypes = [u64, u32, u32, i32, i32, f64, i32, vp, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def normals(seed: int, tensor: int, a: int, row: int, n: int) -> np.ndarray:
    out = np.empty(n, np.float64)
    lib().synth_normal_f64(seed, tensor, a, row, n, _ptr(out))
    return out


def raw_u64(seed: int, tensor: int, a: int, row: int, n: int) -> np.ndarray:
    out = np.empty(n, np.uint64)
    lib().synth_u64(seed, tensor, a, row, n, _ptr(out))
    return out


def x_rows(w: Workload, attempts) -> np.ndarray:
    """bf16 bit patterns [T][H]; row t drawn from attempt ``attempts[t]``."""
    att = np.ascontiguousarray(np.asarray(attempts, np.int32).reshape(-1))
    T = att.shape[0]
    out = np.empty((T, w.H), np.uint16)
    if T:
        lib().synth_x_bf16(w.seed, TENSOR_X, T, w.H, w.x_std, _ptr(att), _ptr(out))
    return out


def block_rows(w: Workload, attempts) -> np.ndarray:
    """Residual-stream rows of a pre-norm block (bf16 bits [T][H]): the rows
    of ``x_rows`` with row t scaled by 2^((t mod 3) - 1), so rows differ in
    magnitude (a power of two keeps every value exact)."""
    b = x_rows(w, attempts)
    f = (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    f = f * np.ldexp(np.float32(1.0), (np.arange(b.shape[0]) % 3 - 1))[:, None].astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def norm_weight(w: Workload) -> np.ndarray:
    """RMSNorm weight [H] fp32: 1 + fp32(N(0, 0.1^2))."""
    out = np.empty((1, w.H), np.float32)
    lib().synth_f32(w.seed, TENSOR_NORM, 0, 1, w.H, 0.1, _ptr(out))
    return (out[0] + np.float32(1.0)).astype(np.float32)


def candidate_rows(w: Workload):
    """The row generator whose draws the margin selection picks from: the
    block input for a pre-norm block, else the layer input."""
    return (lambda a: block_rows(w, a)) if w.prenorm else (lambda a: x_rows(w, a))


def router_weights(w: Workload) -> np.ndarray:
    out = np.empty((w.E, w.H), np.float32)
    lib().synth_f32(w.seed, TENSOR_ROUTER, 0, w.E, w.H, w.router_std, _ptr(out))
    return out


def zipf_bias(w: Workload) -> np.ndarray | None:
    """Per-expert logit offset ln(E * r^-s / H_{E,s}), r = e + 1.

    The log of the Zipf(s) probability of rank r, times E, so an expert of
    average popularity gets 0.  Returned as fp32, or None without skew.
    """
    if w.zipf_s is None:
        return None
    r = np.arange(1, w.E + 1, dtype=np.float64)
    harmonic = np.sum(r ** -w.zipf_s)
    return np.log(w.E * r ** -w.zipf_s / harmonic).astype(np.float32)


def expert_matrix(w: Workload, tensor: int, slot: int, rows: int, K: int):
    q = np.empty((rows, K), np.uint8)
    s = np.empty((rows, K // 32), np.float32)
    lib().synth_fp8_g32(w.seed, tensor, slot, rows, K, w.expert_std, _ptr(q), _ptr(s))
    return q, s


def expert_weights(w: Workload):
    """w13 [E+S][2I][H] (gate rows then up rows), s13 [E+S][2I][H/32],
    w2 [E+S][H][I], s2 [E+S][H][I/32].  Slot E is the shared expert.

    fp8: e4m3fn codes and fp32 scales; mxfp8: e4m3fn codes and E8M0 codes;
    mxfp4: the K axis of w13 and w2 holds bytes of two E2M1 codes (K/2
    bytes), scales are E8M0 codes.  The same normals feed every format."""
    n = w.n_slots
    fmt = w.weight_format
    kb = (lambda K: K // 2) if fmt == "mxfp4" else (lambda K: K)
    st = np.float32 if fmt == "fp8" else np.uint8
    w13 = np.empty((n, 2 * w.I, kb(w.H)), np.uint8)
    s13 = np.empty((n, 2 * w.I, w.H // 32), st)
    w2 = np.empty((n, w.H, kb(w.I)), np.uint8)
    s2 = np.empty((n, w.H, w.I // 32), st)
    L = lib()
    for e in range(n):
        if fmt == "fp8":
            L.synth_fp8_g32(w.seed, TENSOR_W13, e, 2 * w.I, w.H, w.expert_std,
                            _ptr(w13[e]), _ptr(s13[e]))
            L.synth_fp8_g32(w.seed, TENSOR_W2, e, w.H, w.I, w.expert_std,
                            _ptr(w2[e]), _ptr(s2[e]))
        else:
            code = {"mxfp8": 1, "mxfp4": 2}[fmt]
            L.synth_mx_g32(w.seed, TENSOR_W13, e, 2 * w.I, w.H, w.expert_std, code,
                           _ptr(w13[e]), _ptr(s13[e]))
            L.synth_mx_g32(w.seed, TENSOR_W2, e, w.H, w.I, w.expert_std, code,
                           _ptr(w2[e]), _ptr(s2[e]))
    return w13, s13, w2, s2


@dataclasses.dataclass
class Inputs:
    """Host copies of one layer call's inputs, in the library's layouts."""

    workload: Workload
    x: np.ndarray          # [T][H] uint16 (bf16 bits)
    router_w: np.ndarray   # [E][H] fp32
    router_b: np.ndarray | None  # [E] fp32
    w13: np.ndarray
    s13: np.ndarray
    w2: np.ndarray
    s2: np.ndarray
    attempts: np.ndarray   # [T] int32
    norm_w: np.ndarray | None = None  # [H] fp32, pre-norm blocks only


def make_inputs(w: Workload, attempts=None) -> Inputs:
    """All inputs of workload ``w``; ``attempts`` defaults to attempt 0 per row."""
    if attempts is None:
        attempts = np.zeros(w.T, np.int32)
    attempts = np.asarray(attempts, np.int32)
    assert attempts.shape == (w.T,)
    w13, s13, w2, s2 = expert_weights(w)
    return Inputs(w, candidate_rows(w)(attempts), router_weights(w), zipf_bias(w),
                  w13, s13, w2, s2, attempts, norm_weight(w) if w.prenorm else None)
