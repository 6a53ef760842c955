"""The stored per-row draws (tests/golden/attempts.json) are current: a fresh
run of the oracle's margin selection reproduces them."""
import json
import os

import pytest

from moe_decode_layer_amd import synth
from oracle import moe_oracle as O

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "attempts.json")


@pytest.mark.parametrize("i", range(len(synth.WORKLOADS)))
def test_stored_attempts_are_current(i):
    wl = synth.WORKLOADS[i]
    stored = json.load(open(PATH))
    assert stored["margin"] == O.MARGIN and stored["seed"] == wl.seed
    got = O.choose_attempts(wl, lambda a: synth.x_rows(wl, a), synth.router_weights(wl),
                            synth.zipf_bias(wl))
    assert stored["attempts"][wl.name] == [int(a) for a in got]
