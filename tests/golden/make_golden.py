"""Write tests/golden/attempts.json: the draw (attempt) of each x row per workload.

A row of x (of the block input, for pre-norm blocks: the margins are those
of its normalised row) is redrawn until every adjacent gap among its top K+1 sigmoid
scores is at least 1e-3, so that routing has no near-ties.  The decision is
the CPU oracle's (fp64); this script calls only ``oracle/`` and the input
generator.  The bench reads the stored attempts so that it times the same
inputs the parity tests check.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from moe_decode_layer_amd import synth  # noqa: E402
from oracle import moe_oracle as O  # noqa: E402


def attempts_for(wl):
    Wr = synth.router_weights(wl)
    b = synth.zipf_bias(wl)
    nw = synth.norm_weight(wl) if wl.prenorm else None
    return O.attempts_for(wl, synth.candidate_rows(wl), Wr, b, nw)


def main():
    out = {}
    for wl in synth.WORKLOADS + synth.PRENORM + synth.MX + synth.WIDTHS:
        out[wl.name] = [int(a) for a in attempts_for(wl)]
    path = os.path.join(HERE, "attempts.json")
    lines = [f'  "{k}": {json.dumps(v)}' for k, v in out.items()]
    with open(path, "w") as f:
        f.write('{"margin": %r, "seed": 0, "attempts": {\n' % O.MARGIN)
        f.write(",\n".join(lines))
        f.write("\n}}\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
