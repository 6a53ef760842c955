"""HBM traffic of the layer kernel from rocprofv3 counters, calibrated on a copy.

Two steps, each its own process:

1. ``run``: the workload to be profiled.  It makes the bench's inputs, then
   ``--calls`` times sweeps a 1 GiB scratch tensor (evicting the caches, as
   the bench does) and runs the layer once; finally it copies a 256 MiB
   tensor (256 MiB read + 256 MiB written) as the calibration dispatch.
   Run it twice under the profiler, once per counter:

       rocprofv3 --pmc FETCH_SIZE -d OUT/fetch -o f --output-format csv -- \\
           python -m moe_decode_layer_amd.traffic run --workload NAME
       rocprofv3 --pmc WRITE_SIZE -d OUT/write -o w --output-format csv -- \\
           python -m moe_decode_layer_amd.traffic run --workload NAME

2. ``parse``: reads both counter CSVs and writes
   ``profiles/traffic_<workload>.json``: per-launch fetched and written HBM
   bytes of the layer kernel, each scaled by (known copy bytes / what the
   same counter read for the copy), with the hash of the kernel source they
   belong to (the bench ignores the file once the source changes).

       python -m moe_decode_layer_amd.traffic parse --workload NAME \\
           --fetch OUT/fetch --write OUT/write
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SRC = os.path.join(ROOT, "moe_decode_layer_amd", "csrc", "moe_decode.hip")
COPY_BYTES = 256 << 20
KERNEL_NAME = "moe_decode_kernel"


def kernel_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def run(workload: str, calls: int) -> None:
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
    scrub = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    for _ in range(calls):
        scrub.amax()
        (layer.run_block if wl.prenorm else layer.run)(x, y, wl.T)
    torch.cuda.synchronize()
    assert layer.check() == 0
    src = torch.ones(COPY_BYTES // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    scrub.amax()
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    layer.close()
    print(f"ran {calls} calls of {workload} and one {COPY_BYTES >> 20} MiB copy", flush=True)


def _counter_rows(d: str):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _per_dispatch(rows, counter: str):
    """{dispatch id: (kernel name, summed counter value in KiB)}."""
    out = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        did = r.get("Dispatch_Id")
        name = r.get("Kernel_Name", "")
        v = float(r.get("Counter_Value", 0) or 0)
        n, acc = out.get(did, (name, 0.0))
        out[did] = (n, acc + v)
    return out


def _layer_and_copy(d: str, counter: str):
    disp = _per_dispatch(_counter_rows(d), counter)
    layer = [v for n, v in disp.values() if KERNEL_NAME in n]
    copies = [v for n, v in disp.values() if "copy" in n.lower() or "elementwise" in n.lower()]
    if not layer or not copies:
        raise SystemExit(f"{d}: layer dispatches {len(layer)}, copy dispatches {len(copies)}")
    # the calibration copy is the last copy-like dispatch of the run
    return layer, copies[-1]


def parse(workload: str, fetch_dir: str, write_dir: str) -> None:
    lf, cf = _layer_and_copy(fetch_dir, "FETCH_SIZE")
    lw, cw = _layer_and_copy(write_dir, "WRITE_SIZE")
    kib = 1024.0
    f_scale = COPY_BYTES / (cf * kib)
    w_scale = COPY_BYTES / (cw * kib)
    fetch = sorted(v * kib * f_scale for v in lf)
    write = sorted(v * kib * w_scale for v in lw)
    med = lambda a: a[len(a) // 2]
    rec = {
        "workload": workload,
        "kernel_hash": kernel_hash(),
        "calls": len(lf),
        "fetch_bytes_per_launch": med(fetch),
        "write_bytes_per_launch": med(write),
        "hbm_bytes_per_launch": med(fetch) + med(write),
        "fetch_scale": f_scale,
        "write_scale": w_scale,
        "copy_fetch_kib": cf,
        "copy_write_kib": cw,
        "calibration": f"{COPY_BYTES >> 20} MiB device copy: counter KiB vs known bytes",
    }
    out = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    json.dump(rec, open(out, "w"), indent=1)
    print(json.dumps(rec))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--workload", required=True)
    r.add_argument("--calls", type=int, default=5)
    q = sub.add_parser("parse")
    q.add_argument("--workload", required=True)
    q.add_argument("--fetch", required=True)
    q.add_argument("--write", required=True)
    a = ap.parse_args()
    if a.cmd == "run":
        run(a.workload, a.calls)
    else:
        parse(a.workload, a.fetch, a.write)


if __name__ == "__main__":
    main()
