"""CPU oracle of the small-batch MoE decode layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the bench's
CPU-baseline leg use it.  It shares no code with the HIP library.

What it computes is the plain, unfused mixture-of-experts layer that the
fused decode paths on the pages reproduce exactly:

* Router scoring, top-k selection and the weighted reduction over the chosen
  experts plus the shared expert -- "Beyond Day-0: Optimizing DeepSeek-V4.1
  Flash in SGLang", section 2.1 (MoE router / weighted reduction of expert
  outputs / shared-expert addition bullet).
* The placement of token rows into 8-row expert tiles, which must keep the
  router's top-k choices unchanged -- "SGLang's Low-Latency Mode Boosts
  DeepSeek-V4.1-Flash Speed by 1.56x on AMD", section "NVIDIA overlaps the
  dependency chain" (routing without sorting).
* Group-32 FP8 weights -- "Beyond Day-0 ...", section 2.1 (group32 FP8
  weights and scales); the intermediate rounding of the fused SwiGLU --
  same page, section 3.1 (Marlin MoE bullet).
* Routed and shared experts' up/gate and down projections inside one fused
  path -- "FlyDSL Mono Kernels for High-Interactivity LLM Serving in ATOM",
  sections "MiniMax-M3: Connecting Attention and Experts" and
  "DeepSeek-V4.1 in ATOM".

Arithmetic is fp64 throughout except at the two rounding points the layer
defines (the bf16 intermediate h and the bf16 output y).  Matrix products use
numpy's matmul as a library primitive; no blocking, fusion or reordering
beyond the definition.

Readings where the pages are silent (all taken from the workload
definitions, else the plainest reading):
  * score = sigmoid(logit); no grouping; routed scaling 1.0; top-k weights
    renormalised to sum to 1.
  * top-k order: score descending, ties to the lower expert id.
  * SwiGLU: h = silu(g) * u with silu(g) = g * sigmoid(g); gate rows come
    first in the fused gate/up matrix.  Clipped SwiGLU ("Beyond Day-0 ...",
    section 3.1, Marlin MoE bullet; no formula or constant given): with a
    caller's limit L, h = silu(min(g, L)) * clamp(u, -L, L), the gate capped
    from above only (silu is bounded below), the rounding of h unchanged;
    no clipping without a limit.
  * h is rounded to bf16 (nearest even) before the down projection.
  * y = shared + sum_k w_k * o_k in that order, rounded to bf16 from fp64.
  * FP8 is OCP e4m3fn (bias 7, max 448, S.1111.111 is NaN, no infinities);
    dequantised weight = e4m3fn(q) * scale of its 32-element K group.
  * MX weights ("Beyond Day-0 ...", section 3.1: MoE kernels with MXFP4
    weights and BF16 activations; section 2.1: group32 FP8 reorganised for
    MXFP8 kernels), as the OCP Microscaling formats define them: a block of
    32 contiguous K elements shares one E8M0 scale 2^(e - 127) (0xFF NaN);
    MXFP4 elements are E2M1 (bias 1, values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and
    their negatives), two per byte, the lower K index in the low nibble;
    MXFP8 elements are e4m3fn.  Dequantised weight = element * block scale.

The pre-norm block form (input RMSNorm before the router, residual added
after the combine) follows "SGLang's Low-Latency Mode Boosts DeepSeek-V4.1-
Flash Speed by 1.56x on AMD", section "AMD keeps the layer resident" (the
MoE input is normalised and its rows handed on as they become ready), and
"Beyond Day-0 ...", section 2.1 (the next layer's input combined and
normalised right after the MoE).  The pages give no formula; the readings:
  * xn[t] = bf16(x[t] * gamma / sqrt(mean_h x[t][h]^2 + eps)), one rounding
    (the layer's bf16 input), in fp64 here;
  * y[t] = bf16(x[t] + moe(xn)[t]) with the MoE sum unrounded: one rounding
    of the residual stream, where the plain layer rounds the MoE sum alone.

Every function here is pinned by the CPU tests (tests/test_oracle_*.py)
against closed forms, library routines, invariants and brute force.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

TILE_ROWS = 8          # rows per expert tile
GROUP = 32             # K elements per FP8 scale
MARGIN = 1e-3          # minimum adjacent gap among the top K+1 scores


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------
def e4m3fn_value(code: int) -> float:
    """Value of one OCP FP8 E4M3 (fn) code: sign, 4-bit exponent with bias 7,
    3-bit mantissa; exponent 0 is subnormal (m/8 * 2^-6); code S.1111.111 is
    NaN; there are no infinities."""
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3FN = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def e2m1_value(code: int) -> float:
    """Value of one OCP FP4 E2M1 code (the MXFP4 element): sign bit 3,
    exponent bits 2..1 with bias 1, mantissa bit 0; exponent 0 is subnormal
    (m/2); no infinities or NaN."""
    sign = -1.0 if code & 0x8 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    if exp == 0:
        return sign * man * 0.5
    return sign * (1.0 + man / 2.0) * 2.0 ** (exp - 1)


def e8m0_value(code: int) -> float:
    """Value of one OCP E8M0 code (the MX block scale): 2^(code - 127);
    code 0xFF is NaN."""
    return math.nan if code == 0xFF else 2.0 ** (code - 127)


E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E8M0 = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact fp64 values (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_round(v) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value, ties to even, directly
    from fp64 (no intermediate fp32).  bf16 keeps 8 significant bits; its
    smallest step is 2^-133 (subnormals); beyond the largest finite value
    rounding gives +-inf."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)                       # |v| = f * 2^e, f in [0.5, 1)
    step_exp = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(v, -step_exp)), step_exp)
    return np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, v), r)


def bf16_value_to_bits(v: np.ndarray) -> np.ndarray:
    """Bit patterns of values that are already bf16 (exact, no rounding)."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def dequant(q: np.ndarray, s: np.ndarray, fmt: str = "fp8") -> np.ndarray:
    """Expert matrix [..., N, K] -> fp64 weights, one scale per 32 contiguous K.

    fp8   : q [..., N, K] e4m3fn codes, s [..., N, K/32] fp32 scales
    mxfp8 : q [..., N, K] e4m3fn codes, s [..., N, K/32] E8M0 codes
    mxfp4 : q [..., N, K/2] bytes of two E2M1 codes each (element 2j in the
            low nibble, 2j + 1 in the high one), s [..., N, K/32] E8M0 codes
    """
    if fmt == "fp8":
        return E4M3FN[q] * np.repeat(s.astype(np.float64), GROUP, axis=-1)
    scale = np.repeat(E8M0[np.asarray(s, np.uint8)], GROUP, axis=-1)
    if fmt == "mxfp8":
        return E4M3FN[q] * scale
    if fmt == "mxfp4":
        q = np.asarray(q, np.uint8)
        codes = np.stack([q & 0xF, q >> 4], axis=-1).reshape(*q.shape[:-1], 2 * q.shape[-1])
        return E2M1[codes] * scale
    raise ValueError(f"unknown weight format {fmt!r}")


def sigmoid(v: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-np.asarray(v, dtype=np.float64)))


# --------------------------------------------------------------------------
# Router, top-k, placement
# --------------------------------------------------------------------------
def router_logits(X: np.ndarray, Wr: np.ndarray, bias=None) -> np.ndarray:
    """l[t][e] = sum_h X[t][h] * Wr[e][h] (+ bias[e])."""
    l = np.asarray(X, np.float64) @ np.asarray(Wr, np.float64).T
    if bias is not None:
        l = l + np.asarray(bias, np.float64)[None, :]
    return l


def select_topk(scores: np.ndarray, K: int):
    """Per row: the first K experts after ordering by (score desc, id asc);
    weights are the selected scores divided by their sum."""
    T, E = scores.shape
    idx = np.zeros((T, K), np.int32)
    w = np.zeros((T, K), np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-scores[t, e], e))[:K]
        idx[t] = order
        sel = scores[t, order]
        w[t] = sel / sel.sum()
    return idx, w


def topk_margins(scores: np.ndarray, K: int) -> np.ndarray:
    """Smallest gap between adjacent scores among each row's top K+1 (top K
    when K == E).  A row whose gap is >= MARGIN has an unambiguous top-k set
    and order."""
    top = -np.sort(-scores, axis=1)[:, : min(K + 1, scores.shape[1])]
    if top.shape[1] < 2:
        return np.full(scores.shape[0], np.inf)
    return np.min(top[:, :-1] - top[:, 1:], axis=1)


@dataclasses.dataclass
class Placement:
    count: np.ndarray   # [E] rows routed to each expert
    rank: np.ndarray    # [T][K] position of row t among expert idx[t][k]'s rows
    tiles: list         # [(expert, tile j, (rows...))], expert-major, j ascending


def place(idx: np.ndarray, E: int) -> Placement:
    """Canonical tile placement: the rows that chose expert e, in increasing
    row order, fill e's 8-row tiles in turn.  rank(t, k) is the number of
    rows before t that chose the same expert; tile = rank // 8, slot =
    rank % 8."""
    T, K = idx.shape
    rows_of = [[] for _ in range(E)]
    for t in range(T):
        for k in range(K):
            rows_of[int(idx[t, k])].append(t)
    count = np.array([len(r) for r in rows_of], np.int32)
    rank = np.zeros((T, K), np.int32)
    for t in range(T):
        for k in range(K):
            rank[t, k] = rows_of[int(idx[t, k])].index(t)
    tiles = []
    for e in range(E):
        for j in range(0, len(rows_of[e]), TILE_ROWS):
            tiles.append((e, j // TILE_ROWS, tuple(rows_of[e][j:j + TILE_ROWS])))
    return Placement(count, rank, tiles)


# --------------------------------------------------------------------------
# Expert FFN and combine
# --------------------------------------------------------------------------
def expert_ffn(X: np.ndarray, w13q, s13, w2q, s2, limit=None, fmt: str = "fp8") -> np.ndarray:
    """One expert on rows X [n][H]: g/u from the fused gate/up matrix (gate
    rows [0, I), up rows [I, 2I)), h = bf16(silu(g) * u), o = h @ W2^T.
    With a limit L: g -> min(g, L), u -> clamp(u, -L, L) first.  ``fmt``
    names the weight format (see dequant)."""
    I = w13q.shape[0] // 2
    W13 = dequant(w13q, s13, fmt)
    g = X @ W13[:I].T
    u = X @ W13[I:].T
    if limit is not None:
        g = np.minimum(g, float(limit))
        u = np.clip(u, -float(limit), float(limit))
    h = bf16_round(g * sigmoid(g) * u)
    return h @ dequant(w2q, s2, fmt).T


@dataclasses.dataclass
class Result:
    logits: np.ndarray   # [T][E]
    scores: np.ndarray   # [T][E]
    idx: np.ndarray      # [T][K]
    w: np.ndarray        # [T][K]
    placement: Placement
    rows: np.ndarray     # rows for which y was computed
    y: np.ndarray        # [len(rows)][H] fp64, before output rounding
    y_bf16: np.ndarray   # [len(rows)][H] fp64 values of the bf16 output


def forward(inp, rows=None) -> Result:
    """The whole layer for the inputs ``inp`` (see moe_decode_layer_amd.synth.Inputs).

    Routing and placement cover every row; y is computed for ``rows``
    (default: all), so large batches can be checked on a sample.
    """
    wl = inp.workload
    T, H, E, K, S = wl.T, wl.H, wl.E, wl.K, wl.S
    X = bf16_bits_to_f64(inp.x)
    logits = router_logits(X, inp.router_w, inp.router_b)
    scores = sigmoid(logits)
    idx, w = select_topk(scores, K)
    plc = place(idx, E)
    rows = np.arange(T) if rows is None else np.asarray(rows, np.int64)
    pos = {int(t): i for i, t in enumerate(rows)}
    # expert outputs o[(t, slot)] for the requested rows
    o = {}
    need = {}
    for t in rows:
        for k in range(K):
            need.setdefault(int(idx[t, k]), []).append(int(t))
        if S:
            need.setdefault(E, []).append(int(t))
    for e, ts in need.items():
        out = expert_ffn(X[ts], inp.w13[e], inp.s13[e], inp.w2[e], inp.s2[e],
                         getattr(wl, "swiglu_limit", None), getattr(wl, "weight_format", "fp8"))
        for i, t in enumerate(ts):
            o[(t, e)] = out[i]
    y = np.zeros((len(rows), H), np.float64)
    for t in rows:
        acc = o[(int(t), E)].copy() if S else np.zeros(H)
        for k in range(K):
            acc = acc + w[t, k] * o[(int(t), int(idx[t, k]))]
        y[pos[int(t)]] = acc
    return Result(logits, scores, idx, w, plc, rows, y, bf16_round(y))


# --------------------------------------------------------------------------
# Pre-norm block: input RMSNorm and residual
# --------------------------------------------------------------------------
def rmsnorm_bf16(x_bits: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """bf16 bits of x * gamma / sqrt(mean(x^2) + eps) per row of x [T][H]
    (bf16 bits), computed in fp64 and rounded once."""
    X = bf16_bits_to_f64(x_bits)
    ms = np.mean(X * X, axis=1, keepdims=True)
    xn = X * (1.0 / np.sqrt(ms + float(eps))) * np.asarray(gamma, np.float64)[None, :]
    return bf16_value_to_bits(bf16_round(xn))


@dataclasses.dataclass
class BlockResult:
    xn: np.ndarray       # [T][H] bf16 bits: the rows the MoE layer ran on
    moe: Result          # the plain layer on xn
    y: np.ndarray        # [len(rows)][H] fp64 x + moe, before output rounding
    y_bf16: np.ndarray   # [len(rows)][H] fp64 values of the bf16 output


def forward_block(inp, rows=None) -> BlockResult:
    """x -> xn = RMSNorm(x) -> the layer -> y = bf16(x + layer(xn)).  ``inp``
    carries the block input in ``x`` and the norm weight and epsilon in
    ``norm_w`` / ``workload.norm_eps``."""
    xn = rmsnorm_bf16(inp.x, inp.norm_w, inp.workload.norm_eps)
    res = forward(dataclasses.replace(inp, x=xn), rows)
    y = bf16_bits_to_f64(inp.x)[res.rows] + res.y
    return BlockResult(xn, res, y, residual_add(inp.x[res.rows], res.y))


def residual_add(x_bits: np.ndarray, moe: np.ndarray) -> np.ndarray:
    """The block output bf16(x + moe): the residual row x (bf16 bits) plus the
    layer's unrounded output, rounded once to bf16 from the exact fp64 sum
    (the residual stream is rounded once, not after a rounded MoE output)."""
    return bf16_round(bf16_bits_to_f64(x_bits) + np.asarray(moe, np.float64))


# --------------------------------------------------------------------------
# Input selection with routing margins
# --------------------------------------------------------------------------
def choose_attempts(wl, x_rows, router_w, router_b, max_attempts: int = 1000) -> np.ndarray:
    """Attempt index per row such that every adjacent gap among the row's
    top K+1 sigmoid scores is at least MARGIN.  ``x_rows(attempts)`` draws
    the candidate rows (bf16 bits).  Fails loudly after ``max_attempts``."""
    att = np.zeros(wl.T, np.int32)
    todo = np.arange(wl.T)
    while todo.size:
        X = bf16_bits_to_f64(x_rows(att))
        s = sigmoid(router_logits(X[todo], router_w, router_b))
        bad = todo[topk_margins(s, wl.K) < MARGIN]
        if bad.size and att[bad].max() + 1 >= max_attempts:
            raise RuntimeError(f"{wl.name}: no row with top-k margins after {max_attempts} draws")
        att[bad] += 1
        todo = bad
    return att


def choose_attempts_block(wl, x_rows, norm_w, router_w, router_b,
                          max_attempts: int = 1000) -> np.ndarray:
    """choose_attempts for a pre-norm block: the margins are those of the
    normalised rows the router sees."""
    return choose_attempts(wl, lambda a: rmsnorm_bf16(x_rows(a), norm_w, wl.norm_eps),
                           router_w, router_b, max_attempts)


def attempts_for(wl, rows, router_w, router_b, norm_w=None) -> np.ndarray:
    """The margin selection that fits the workload (plain layer or block)."""
    if getattr(wl, "prenorm", False):
        return choose_attempts_block(wl, rows, norm_w, router_w, router_b)
    return choose_attempts(wl, rows, router_w, router_b)
