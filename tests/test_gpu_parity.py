"""GPU parity: the HIP layer, called through the C ABI, against the CPU oracle.

Bars: top-k indices, placement ranks and expert counts bit-exact; top-k
weights within 1e-5; logits within 1e-4 relative; y (bf16) within
max|d|/max|o| <= 1e-2 and sum|d|/sum|o| <= 2e-3 of the oracle's bf16 y.
Inputs are the seeded synthetic workloads (rows redrawn for top-k margins,
tests/golden/attempts.json).  y is compared on every row, the 384- and
512-row batches included.
"""
import json
import os

import numpy as np
import pytest
import torch

from checks import MAX_REL, MEAN_REL, check_placement, output_errors
from moe_decode_layer_amd import binding, device, synth
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "attempts.json")))
_cache = {}


def inputs_for(wl):
    if wl.name not in _cache:
        att = GOLDEN["attempts"].get(wl.name)
        if att is None:
            att = O.attempts_for(wl, synth.candidate_rows(wl), synth.router_weights(wl),
                                 synth.zipf_bias(wl), synth.norm_weight(wl) if wl.prenorm else None)
        _cache.clear()
        _cache[wl.name] = synth.make_inputs(wl, att)
    return _cache[wl.name]


def check_against_oracle(wl, inp, out, rows=None, T=None):
    T = wl.T if T is None else T
    ref = O.forward(inp, rows)
    assert np.array_equal(out["topk_idx"], ref.idx), "top-k indices differ"
    assert np.array_equal(out["expert_count"], ref.placement.count), "expert counts differ"
    assert np.array_equal(out["pair_rank"], ref.placement.rank), "placement ranks differ"
    check_placement(out["topk_idx"], out["pair_rank"], out["expert_count"], wl.E)
    assert np.abs(out["topk_w"] - ref.w).max() <= 1e-5
    l_err = np.abs(out["logits"] - ref.logits).max() / np.abs(ref.logits).max()
    assert l_err <= 1e-4, f"logits rel err {l_err}"
    y = O.bf16_bits_to_f64(out["y"])[ref.rows]
    mx, mean = output_errors(y, ref.y_bf16)
    print(f"{wl.name}: max_rel {mx:.3e} mean_rel {mean:.3e} (rows {len(ref.rows)})")
    assert mx <= MAX_REL and mean <= MEAN_REL, (mx, mean)
    return ref


@pytest.mark.parametrize("i", range(len(synth.WORKLOADS)), ids=[w.name for w in synth.WORKLOADS])
def test_workload_parity(i):
    wl = synth.WORKLOADS[i]
    print(f"case {wl.name}", flush=True)
    inp = inputs_for(wl)
    layer = device.make_layer(inp)
    out = device.run_once(layer, inp.x, wl.E, wl.K)
    check_against_oracle(wl, inp, out)
    # a second run on the same handle gives the same bits (counters were reset,
    # the combine order is fixed)
    again = device.run_once(layer, inp.x, wl.E, wl.K)
    assert np.array_equal(again["y"], out["y"])
    layer.close()


SMALL = [
    synth.Workload("t20_h128_e8_k8_s1", T=20, H=128, E=8, K=8, S=1, I=64),      # K = E
    synth.Workload("t3_h64_e1_k1_s0", T=3, H=64, E=1, K=1, S=0, I=64),          # one expert
    synth.Workload("t70_h192_e4_k2_s1", T=70, H=192, E=4, K=2, S=1, I=192),     # ragged H, 2 chunks
    synth.Workload("t200_h256_e4_k2_s0", T=200, H=256, E=4, K=2, S=0, I=128),   # 100 rows/expert
    synth.Workload("t33_h320_e64_k6_s1", T=33, H=320, E=64, K=6, S=1, I=128, zipf_s=1.2),
    synth.Workload("t9_h4096_e256_k8_s1", T=9, H=4096, E=256, K=8, S=1, I=512),
    # the real per-GPU intermediate width of the pages' model (18 scale groups),
    # run without padding to 640: the general items, x in LDS
    synth.Workload("t6_h4096_e256_k8_s1_i576", T=6, H=4096, E=256, K=8, S=1, I=576),
    # the same width at larger batches (64 rows: Zipf-skewed, hot experts over
    # 32 rows; 384 rows)
    synth.Workload("t64_h4096_e256_k8_s1_i576", T=64, H=4096, E=256, K=8, S=1, I=576, zipf_s=1.2),
    synth.Workload("t384_h4096_e256_k8_s1_i576", T=384, H=4096, E=256, K=8, S=1, I=576),
    # the per-GPU width of TP8 (not a multiple of 64: run padded to 320 with
    # zero weights), small and larger batches
    synth.Workload("t6_h4096_e256_k8_s1_i288", T=6, H=4096, E=256, K=8, S=1, I=288),
    synth.Workload("t40_h4096_e256_k8_s1_i288", T=40, H=4096, E=256, K=8, S=1, I=288, zipf_s=1.2),
    synth.Workload("t20_h128_e8_k8_s1_i96", T=20, H=128, E=8, K=8, S=1, I=96),
    # 576 padded to 640 (the pages' padded width): wide items with 10 down K tiles
    synth.Workload("t40_h4096_e256_k8_s1_i640", T=40, H=4096, E=256, K=8, S=1, I=640, zipf_s=1.2),
]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_edge_shapes(wl):
    print(f"case {wl.name}", flush=True)
    inp = inputs_for(wl)
    layer = device.make_layer(inp)
    out = device.run_once(layer, inp.x, wl.E, wl.K)
    check_against_oracle(wl, inp, out)
    layer.close()


@pytest.mark.parametrize("wl", [synth.WORKLOADS[1], SMALL[0]], ids=lambda w: w.name)
def test_cooperative_launch_matches_the_plain_launch(wl):
    """MOE_FLAG_COOPERATIVE (the runtime guarantees the grid co-resident or
    refuses the launch): the same bits as the plain launch, run after run, and
    the oracle's bars (6 rows: the full-tile variant; 20 rows: router tiles
    and the distributed top-k)."""
    print(f"case {wl.name} cooperative", flush=True)
    inp = inputs_for(wl)
    plain = device.make_layer(inp)
    coop = device.make_layer(inp, cooperative=True)
    want = device.run_once(plain, inp.x, wl.E, wl.K)
    check_against_oracle(wl, inp, want)
    for _ in range(3):
        got = device.run_once(coop, inp.x, wl.E, wl.K)
        for key in ("y", "topk_idx", "pair_rank", "expert_count"):
            assert np.array_equal(got[key], want[key]), key
    plain.close()
    coop.close()


def test_ragged_T_on_one_handle():
    wl = synth.WORKLOADS[1]
    print(f"case ragged T on {wl.name}", flush=True)
    inp = inputs_for(wl)
    layer = device.make_layer(inp, max_tokens=wl.T)
    for T in (1, 4, 6, 2):
        sub = synth.Inputs(wl.with_rows(T), inp.x[:T], inp.router_w, inp.router_b, inp.w13,
                           inp.s13, inp.w2, inp.s2, inp.attempts[:T])
        out = device.run_once(layer, sub.x, wl.E, wl.K)
        check_against_oracle(sub.workload, sub, out)
    layer.close()


@pytest.mark.parametrize("name", ["verify_t384_h4096_e256_k8_s1", "verify_t384_h4096_e256_k8_s1_i576"])
def test_ragged_T_on_one_wide_handle(name):
    """Batches above 16 rows take the wide items (32-row expert ranges, 4-block
    gate/up and 512-row down items, at I = 512 or 576): the smallest such
    batch, ragged expert ranges and the full 384 rows, on one handle."""
    wl = synth.BY_NAME[name]
    inp = inputs_for(wl)
    layer = device.make_layer(inp, max_tokens=wl.T)
    for T in (17, 45, 200, wl.T):
        print(f"case wide T={T} on {wl.name}", flush=True)
        sub = synth.Inputs(wl.with_rows(T), inp.x[:T], inp.router_w, inp.router_b, inp.w13,
                           inp.s13, inp.w2, inp.s2, inp.attempts[:T])
        out = device.run_once(layer, sub.x, wl.E, wl.K)
        check_against_oracle(sub.workload, sub, out)
    layer.close()


def test_maximum_batch_on_the_wide_path():
    """512 rows (the supported maximum): eight 64-row bitmap chunks, the
    widest LDS layout of the wide items, checked on every row."""
    wl = synth.Workload("t512_h4096_e256_k8_s1", T=512, H=4096, E=256, K=8, S=1, I=512)
    print(f"case {wl.name}", flush=True)
    inp = inputs_for(wl)
    layer = device.make_layer(inp)
    out = device.run_once(layer, inp.x, wl.E, wl.K)
    check_against_oracle(wl, inp, out)
    layer.close()


@pytest.mark.parametrize("wi,Ts", [(1, (6, 1, 3, 6, 2, 5)), (4, (384, 17, 200, 64, 33))],
                         ids=["small_batches", "wide_batches"])
def test_many_runs_on_one_handle_repeat_bit_for_bit(wi, Ts):
    """Forty runs on one handle with the row count changing every run: every
    run's y equals, bit for bit, the first run with the same rows (the epoch
    tags, the alternating counter blocks and the per-run clearing leave no
    state behind), and the first run of each row count matches the oracle."""
    wl = synth.WORKLOADS[wi]
    inp = inputs_for(wl)
    layer = device.make_layer(inp, max_tokens=wl.T)
    first = {}
    for i in range(40):
        T = Ts[i % len(Ts)]
        out = device.run_once(layer, np.ascontiguousarray(inp.x[:T]), wl.E, wl.K, debug=(T not in first))
        if T not in first:
            print(f"case {wl.name} T={T}", flush=True)
            sub = synth.Inputs(wl.with_rows(T), inp.x[:T], inp.router_w, inp.router_b, inp.w13,
                               inp.s13, inp.w2, inp.s2, inp.attempts[:T])
            check_against_oracle(sub.workload, sub, out)
            first[T] = out["y"]
        else:
            assert np.array_equal(out["y"], first[T]), f"run {i} (T={T}) differs from the first"
    layer.close()


def test_two_handles_interleaved_on_one_stream():
    """Two handles (different shapes and variants) alternating on one stream
    keep separate counters and tags: each one's output is its own first
    output, bit for bit, run after run."""
    wa, wb = synth.WORKLOADS[1], synth.WORKLOADS[0]
    ia = synth.make_inputs(wa, GOLDEN["attempts"].get(wa.name))
    ib = synth.make_inputs(wb, GOLDEN["attempts"].get(wb.name))
    la, lb = device.make_layer(ia), device.make_layer(ib)
    ya = device.run_once(la, ia.x, wa.E, wa.K, debug=False)["y"]
    yb = device.run_once(lb, ib.x, wb.E, wb.K, debug=False)["y"]
    dev = torch.device("cuda", 0)
    xa, xb = device.to_device(ia.x, dev), device.to_device(ib.x, dev)
    outs = []
    for _ in range(6):
        for layer, x, T in ((la, xa, wa.T), (lb, xb, wb.T)):
            y = torch.empty_like(x)
            layer.run(x, y, T)
            outs.append(y)
    assert la.check() == binding.MOE_OK and lb.check() == binding.MOE_OK
    for i, y in enumerate(outs):
        ref = ya if i % 2 == 0 else yb
        assert np.array_equal(y.cpu().numpy().view(np.uint16), ref), f"run {i} differs"
    la.close()
    lb.close()


def test_zero_rows_is_a_noop():
    wl = synth.WORKLOADS[0]
    inp = inputs_for(wl)
    layer = device.make_layer(inp)
    dev = torch.device("cuda", 0)
    x = device.to_device(inp.x, dev)
    y = torch.full_like(x, 7)
    layer.run(x, y, 0)
    assert layer.check() == binding.MOE_OK
    assert torch.all(y == 7)
    layer.close()


def test_row_permutation_and_single_rows_are_bit_identical():
    wl = synth.WORKLOADS[1]
    inp = inputs_for(wl)
    layer = device.make_layer(inp)
    base = device.run_once(layer, inp.x, wl.E, wl.K, debug=False)["y"]
    perm = np.array([3, 0, 5, 1, 4, 2])
    permuted = device.run_once(layer, np.ascontiguousarray(inp.x[perm]), wl.E, wl.K, debug=False)["y"]
    assert np.array_equal(permuted, base[perm])
    for t in range(wl.T):
        one = device.run_once(layer, np.ascontiguousarray(inp.x[t:t + 1]), wl.E, wl.K, debug=False)["y"]
        assert np.array_equal(one[0], base[t]), f"row {t} alone differs from the batch"
    layer.close()


def test_power_of_two_down_scales_scale_y_exactly():
    wl = synth.WORKLOADS[0]
    inp = inputs_for(wl)
    layer = device.make_layer(inp)
    base = device.run_once(layer, inp.x, wl.E, wl.K, debug=False)["y"]
    layer.close()
    scaled = synth.Inputs(wl, inp.x, inp.router_w, inp.router_b, inp.w13, inp.s13, inp.w2,
                          (inp.s2 * np.float32(0.25)).astype(np.float32), inp.attempts)
    layer = device.make_layer(scaled)
    got = device.run_once(layer, inp.x, wl.E, wl.K, debug=False)["y"]
    layer.close()
    assert np.array_equal(O.bf16_bits_to_f64(got), 0.25 * O.bf16_bits_to_f64(base))


def test_expired_waits_report_timeout_and_the_next_run_recovers():
    """Deadline path, forced from the host: every in-kernel wait of the run gives
    up at once.  The kernel must end (no hang), report MOE_ERR_TIMEOUT through
    check, clear it, and leave the handle fit for the next run."""
    wl = synth.WORKLOADS[1]
    print(f"case expire_waits on {wl.name}", flush=True)
    inp = inputs_for(wl)
    layer = device.make_layer(inp)
    dev = torch.device("cuda", 0)
    x = device.to_device(inp.x, dev)
    y = torch.empty_like(x)
    for _ in range(2):
        layer.run(x, y, wl.T, {"expire_waits": 1})
        assert layer.check() == binding.MOE_ERR_TIMEOUT
    assert layer.check() == binding.MOE_OK
    out = device.run_once(layer, inp.x, wl.E, wl.K)
    check_against_oracle(wl, inp, out)
    layer.close()


def _check_routing_in_kernel_precision(wl, inp, out):
    """Routing decided in the precision the kernel decides it in: the oracle's
    selection and placement applied to the kernel's own fp32 logits, which
    are themselves checked against the oracle's."""
    ref_l = O.router_logits(O.bf16_bits_to_f64(inp.x), inp.router_w, inp.router_b)
    scale = max(np.abs(ref_l).max(), 1e-30)
    assert np.abs(out["logits"] - ref_l).max() / scale <= 1e-4
    idx, w = O.select_topk(O.sigmoid(out["logits"].astype(np.float64)), wl.K)
    assert np.array_equal(out["topk_idx"], idx), "top-k indices differ"
    assert np.abs(out["topk_w"] - w).max() <= 1e-5
    plc = O.place(idx, wl.E)
    assert np.array_equal(out["expert_count"], plc.count)
    assert np.array_equal(out["pair_rank"], plc.rank)
    check_placement(out["topk_idx"], out["pair_rank"], out["expert_count"], wl.E)


def test_exactly_tied_router_rows_break_ties_by_expert_id():
    """Experts 2j and 2j+1 get identical router rows (and biases), so every
    row's logits come in exactly equal pairs: the filtered selection must
    order each tied pair by expert id, as the round-by-round one does."""
    wl = synth.WORKLOADS[1]
    print(f"case tied router rows on {wl.name}", flush=True)
    inp = inputs_for(wl)
    rw = inp.router_w.copy()
    rw[1::2] = rw[0::2]
    rb = None if inp.router_b is None else inp.router_b.copy()
    if rb is not None:
        rb[1::2] = rb[0::2]
    tied = synth.Inputs(wl, inp.x, rw, rb, inp.w13, inp.s13, inp.w2, inp.s2, inp.attempts)
    layer = device.make_layer(tied)
    out = device.run_once(layer, tied.x, wl.E, wl.K)
    layer.close()
    lg = out["logits"]
    assert np.array_equal(lg[:, 0::2], lg[:, 1::2]), "tied experts got different logits"
    _check_routing_in_kernel_precision(wl, tied, out)
    # some row selects both members of a tied pair (else the case tests nothing)
    sel = out["topk_idx"]
    assert any(len(set(sel[t] // 2)) < wl.K for t in range(wl.T))


def test_all_equal_logits_select_the_lowest_expert_ids():
    """A zero router (and bias) makes all logits equal: every row selects
    experts 0..K-1 in order with equal weights (the many-candidates path)."""
    wl = synth.WORKLOADS[1]
    print(f"case all-equal logits on {wl.name}", flush=True)
    inp = inputs_for(wl)
    zero = synth.Inputs(wl, inp.x, np.zeros_like(inp.router_w),
                        None if inp.router_b is None else np.zeros_like(inp.router_b),
                        inp.w13, inp.s13, inp.w2, inp.s2, inp.attempts)
    layer = device.make_layer(zero)
    out = device.run_once(layer, zero.x, wl.E, wl.K)
    layer.close()
    assert np.all(out["logits"] == 0.0)
    assert np.array_equal(out["topk_idx"], np.tile(np.arange(wl.K, dtype=np.int32), (wl.T, 1)))
    assert np.abs(out["topk_w"] - 1.0 / wl.K).max() <= 1e-6
    _check_routing_in_kernel_precision(wl, zero, out)


@pytest.mark.parametrize("name", ["verify_t6_h4096_e256_k8_s1", "verify_t6_h4096_e256_k8_s1_mxfp4",
                                  "zipf_t64_h4096_e256_k8_s1"])
def test_relabelled_experts_give_the_same_y(name):
    """Routed expert e moved to id p[e] (router row, bias and packed weights
    together): the kernel selects p[idx] and returns the same y bit for bit,
    since every logit and every expert output is formed in the same order
    wherever its expert sits.  Checks the expert id -> weight slot mapping of
    the router tiles, the placement and the packed layouts."""
    wl = synth.BY_NAME[name]
    print(f"case relabelled experts {name}", flush=True)
    inp = inputs_for(wl)
    layer = device.make_layer(inp)
    base = device.run_once(layer, inp.x, wl.E, wl.K)
    layer.close()
    p = np.random.default_rng(5).permutation(wl.E)
    moved = synth.Inputs(wl, inp.x, np.empty_like(inp.router_w), None, np.empty_like(inp.w13),
                         np.empty_like(inp.s13), np.empty_like(inp.w2), np.empty_like(inp.s2), inp.attempts)
    moved.router_w[p] = inp.router_w
    if inp.router_b is not None:
        moved.router_b = np.empty_like(inp.router_b)
        moved.router_b[p] = inp.router_b
    for field in ("w13", "s13", "w2", "s2"):
        src, dst = getattr(inp, field), getattr(moved, field)
        dst[p] = src[:wl.E]
        dst[wl.E:] = src[wl.E:]                      # the shared expert keeps slot E
    layer = device.make_layer(moved)
    got = device.run_once(layer, inp.x, wl.E, wl.K)
    layer.close()
    assert np.array_equal(got["topk_idx"], p[base["topk_idx"]])
    assert np.array_equal(got["topk_w"], base["topk_w"])
    assert np.array_equal(got["y"], base["y"])
