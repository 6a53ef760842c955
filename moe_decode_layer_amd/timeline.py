"""Phase breakdown of one layer call from the kernel's per-workgroup timeline.

The debug ``trace`` buffer (include/moe_decode.h) records, for every
workgroup, its entry and exit time and, per item, the item's kind, when the
workgroup got it, when its inputs were ready and when it was done (device wall
clock, 100 MHz).  This script runs a workload a few times (cold caches: a
1 GiB read-only sweep before each call, as in the bench), keeps the median
call by kernel span, and prints when each kind of item started and finished
across the grid, and the HBM rate of the expert items while they streamed.

    python -m moe_decode_layer_amd.timeline --workload verify_t6_h4096_e256_k8_s1

The same numbers, summarised, are committed under profiles/ as the phase
breakdown of a workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

KINDS = {0: "router", 1: "shared gate/up", 2: "top-k", 3: "shared down", 4: "routed gate/up",
         5: "routed down", 6: "exit", 7: "combine", 11: "norm row"}
TICK_US = 0.01          # the wall clock runs at 100 MHz


def collect(workload: str, calls: int, cap: int = 64):
    sys.path.insert(0, ROOT)
    import torch

    from moe_decode_layer_amd import device, synth
    wl = synth.BY_NAME[workload]
    att = json.load(open(os.path.join(ROOT, "tests", "golden", "attempts.json")))["attempts"].get(wl.name)
    inp = synth.make_inputs(wl, att)
    dev = torch.device("cuda", 0)
    layer = device.make_layer(inp)
    x = device.to_device(inp.x, dev)
    y = torch.empty_like(x)
    dbg = device.debug_buffers(wl.T, wl.E, wl.K, dev)
    run = layer.run_block if wl.prenorm else layer.run
    run(x, y, wl.T, dbg)
    assert layer.check() == 0
    counts = dbg["expert_count"].cpu().numpy()
    experts = int((counts > 0).sum()) + wl.S
    scrub = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    blocks = 4096
    traces = []
    for _ in range(calls):
        tr = torch.zeros((blocks, 1 + cap, 4), dtype=torch.int64, device=dev)
        scrub.amax()
        torch.cuda.synchronize()
        run(x, y, wl.T, {"trace": tr})
        torch.cuda.synchronize()
        assert layer.check() == 0
        traces.append(tr.cpu().numpy())
    layer.close()
    return wl, experts, traces


def summarise(wl, experts: int, tr: np.ndarray) -> dict:
    G = int(tr[0, 0, 3])
    tr = tr[:G]
    t0 = tr[:, 0, 0].min()
    entry = (tr[:, 0, 0] - t0) * TICK_US
    exit_ = (tr[:, 0, 1] - t0) * TICK_US
    ev = []
    for b in range(G):
        n = min(int(tr[b, 0, 2]), tr.shape[1] - 1)
        for i in range(n):
            w = tr[b, 1 + i]
            kind = int(w[0] >> 32)
            if kind in KINDS:
                ev.append((kind, (w[1] - t0) * TICK_US, (w[2] - t0) * TICK_US, (w[3] - t0) * TICK_US))
    ev = np.array(ev) if ev else np.zeros((0, 4))
    # per workgroup: time inside items, gaps between consecutive items, waits
    busy, gaps = [], []
    for b in range(G):
        n = min(int(tr[b, 0, 2]), tr.shape[1] - 1)
        rows = [tr[b, 1 + i] for i in range(n) if int(tr[b, 1 + i][0] >> 32) in KINDS]
        rows = [r for r in rows if int(r[0] >> 32) != 6]
        busy.append(sum((r[3] - r[1]) for r in rows) * TICK_US)
        gaps += [(rows[i + 1][1] - rows[i][3]) * TICK_US for i in range(len(rows) - 1)]
    out = {"workgroups": G, "span_us": float(exit_.max() - entry.min()),
           "busy_fraction": float(np.sum(busy) / (G * (exit_.max() - entry.min()))),
           "median_gap_between_items_us": float(np.median(gaps)) if gaps else 0.0,
           "mean_gap_between_items_us": float(np.mean(gaps)) if gaps else 0.0,
           "entry_us": [float(np.percentile(entry, q)) for q in (0, 50, 100)],
           "exit_us": [float(np.percentile(exit_, q)) for q in (0, 50, 100)], "kinds": {}}
    for k, name in KINDS.items():
        sel = ev[ev[:, 0] == k] if len(ev) else ev
        if not len(sel):
            continue
        out["kinds"][name] = {
            "items": int(len(sel)),
            "first_start_us": float(sel[:, 1].min()),
            "median_start_us": float(np.median(sel[:, 1])),
            "median_ready_us": float(np.median(sel[:, 2])),
            "last_end_us": float(sel[:, 3].max()),
            "median_duration_us": float(np.median(sel[:, 3] - sel[:, 1])),
            "median_wait_us": float(np.median(sel[:, 2] - sel[:, 1])),
            "median_after_ready_us": float(np.median(sel[:, 3] - sel[:, 2])),
        }
    # routing inside each workgroup: kind 8 = {start, gather begins, top-k
    # done; placement time}, kind 9 = {logits in LDS, row 0 selected, all
    # rows selected}
    # (all workgroups, then split by the kind of the workgroup's first item:
    # router, shared gate/up, or none before the routing)
    def routing_of(sel):
        r8, r9 = [], []
        for b in sel:
            n = min(int(tr[b, 0, 2]), tr.shape[1] - 1)
            for i in range(n):
                w = tr[b, 1 + i]
                k = int(w[0] >> 32)
                if k == 8:
                    # a stamp of 0: that phase does not exist on this path
                    go = (w[2] - t0) * TICK_US if w[2] else np.nan
                    r8.append(((w[1] - t0) * TICK_US, go, (w[3] - t0) * TICK_US,
                               ((w[3] - t0) + (int(w[0]) & 0xffffffff)) * TICK_US))
                elif k == 9 and w[1]:
                    # low 16 bits: shader-clock cycles from logits in LDS to all rows selected
                    r9.append(((w[1] - t0) * TICK_US, (w[2] - t0) * TICK_US, (w[3] - t0) * TICK_US,
                               int(w[0]) & 0xffff, (w[3] - w[1]) * TICK_US))
        if not r8:
            return None
        r8 = np.array(r8)
        r = {"workgroups": len(r8), "median_start_us": float(np.median(r8[:, 0])),
             "median_gather_begins_us": float(np.nanmedian(r8[:, 1])) if np.isfinite(r8[:, 1]).any() else float("nan"),
             "median_topk_done_us": float(np.median(r8[:, 2])),
             "median_placement_done_us": float(np.median(r8[:, 3])),
             "last_placement_done_us": float(r8[:, 3].max())}
        if r9:
            r9 = np.array(r9)
            r.update({"median_logits_in_lds_us": float(np.median(r9[:, 0])),
                      "median_row0_selected_us": float(np.median(r9[:, 1])),
                      "median_rows_selected_us": float(np.median(r9[:, 2])),
                      # top-k span in shader cycles and wall time: their ratio is the clock
                      "median_topk_cycles": float(np.median(r9[:, 3])),
                      "median_topk_wall_us": float(np.median(r9[:, 4]))})
        return r

    first = {}
    for b in range(G):
        n = min(int(tr[b, 0, 2]), tr.shape[1] - 1)
        k = int(tr[b, 1, 0] >> 32) if n > 0 else -1
        first.setdefault({0: "router", 1: "shared gate/up"}.get(k, "none"), []).append(b)
    r = routing_of(range(G))
    if r:
        out["routing"] = r
        out["routing_by_first_item"] = {k: routing_of(v) for k, v in first.items() if routing_of(v)}
    # expert streaming: from the first routed gate/up start to the last down end
    ks = out["kinds"]
    if "routed gate/up" in ks and "routed down" in ks:
        a = min(ks["routed gate/up"]["first_start_us"], ks.get("shared gate/up", {}).get("first_start_us", 1e9))
        z = max(ks["routed down"]["last_end_us"], ks.get("shared down", {}).get("last_end_us", 0))
        gu_end = ks["routed gate/up"]["last_end_us"]
        out["expert_window_us"] = [a, z]
        out["expert_bytes"] = experts * wl.expert_bytes()
        out["expert_window_gbs"] = experts * wl.expert_bytes() / ((z - a) * 1e-6) / 1e9
        out["gate_up_end_us"] = gu_end
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="verify_t6_h4096_e256_k8_s1")
    ap.add_argument("--calls", type=int, default=7)
    ap.add_argument("--json", default=None, help="also write the summary of the median call here")
    ap.add_argument("--raw", default=None, help="also save every call's trace array here (.npy)")
    args = ap.parse_args()
    wl, experts, traces = collect(args.workload, args.calls)
    if args.raw:
        G = int(traces[0][0, 0, 3])
        np.save(args.raw, np.stack([t[:G] for t in traces]))
    sums = [summarise(wl, experts, t) for t in traces]
    spans = [s["span_us"] for s in sums]
    med = sums[int(np.argsort(spans)[len(spans) // 2])]
    med["spans_us_all_calls"] = spans
    med["workload"] = wl.name
    med["experts_streamed"] = experts
    print(f"{wl.name}: kernel span (first entry to last exit) median {np.median(spans):.1f} us "
          f"over {len(spans)} calls; {med['workgroups']} workgroups")
    print(f"  entry  {med['entry_us'][0]:7.1f} .. {med['entry_us'][2]:7.1f} us")
    for name, k in med["kinds"].items():
        print(f"  {name:15s} {k['items']:5d} items  start {k['first_start_us']:6.1f} (median "
              f"{k['median_start_us']:6.1f})  ready median {k['median_ready_us']:6.1f}  "
              f"last end {k['last_end_us']:6.1f}  median item {k['median_duration_us']:5.2f} us "
              f"(wait {k['median_wait_us']:5.2f}, then {k['median_after_ready_us']:5.2f})")
    print(f"  workgroups busy {100 * med['busy_fraction']:.0f}% of the span; gap between items "
          f"median {med['median_gap_between_items_us']:.2f}, mean {med['mean_gap_between_items_us']:.2f} us")
    if "routing" in med:
        r = med["routing"]
        print(f"  routing (medians): start {r['median_start_us']:.1f}, gather begins "
              f"{r['median_gather_begins_us']:.1f}, logits in LDS {r.get('median_logits_in_lds_us', float('nan')):.1f}, "
              f"row 0 selected {r.get('median_row0_selected_us', float('nan')):.1f}, all rows selected "
              f"{r.get('median_rows_selected_us', float('nan')):.1f}, top-k done {r['median_topk_done_us']:.1f}, "
              f"placement done {r['median_placement_done_us']:.1f} (last {r['last_placement_done_us']:.1f}) us")
        for k, g in med.get("routing_by_first_item", {}).items():
            print(f"    first item {k:15s} ({g['workgroups']:3d}): start {g['median_start_us']:.1f}, gather "
                  f"{g['median_gather_begins_us']:.1f}, logits {g.get('median_logits_in_lds_us', float('nan')):.1f}, "
                  f"row 0 {g.get('median_row0_selected_us', float('nan')):.1f}, top-k {g['median_topk_done_us']:.1f}, "
                  f"placement {g['median_placement_done_us']:.1f}; top-k {g.get('median_topk_cycles', 0):.0f} cycles "
                  f"in {g.get('median_topk_wall_us', 0):.2f} us")
    if "expert_window_us" in med:
        a, z = med["expert_window_us"]
        print(f"  experts stream {a:.1f} .. {z:.1f} us: {med['expert_bytes'] / 1e6:.1f} MB at "
              f"{med['expert_window_gbs']:.0f} GB/s; last gate/up ends {med['gate_up_end_us']:.1f} us")
    print(f"  exit   {med['exit_us'][0]:7.1f} .. {med['exit_us'][2]:7.1f} us")
    if args.json:
        with open(args.json, "w") as f:
            json.dump(med, f, indent=1)


if __name__ == "__main__":
    main()
