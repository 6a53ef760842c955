"""The stored per-row draws (tests/golden/attempts.json) are current: a fresh
run of the oracle's margin selection reproduces them."""
import json
import os

import pytest

from moe_decode_layer_amd import synth
from oracle import moe_oracle as O

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "attempts.json")


ALL = synth.WORKLOADS + synth.PRENORM + synth.MX + synth.WIDTHS


@pytest.mark.parametrize("i", range(len(ALL)))
def test_stored_attempts_are_current(i):
    wl = ALL[i]
    stored = json.load(open(PATH))
    assert stored["margin"] == O.MARGIN and stored["seed"] == wl.seed
    got = O.attempts_for(wl, synth.candidate_rows(wl), synth.router_weights(wl),
                         synth.zipf_bias(wl), synth.norm_weight(wl) if wl.prenorm else None)
    assert stored["attempts"][wl.name] == [int(a) for a in got]
