"""Pins of the oracle's frame routing (NanoKV appendix Table 7) and anchor
precision rule (TempoKV section 3.3): the deployed rules worked by hand."""
import json
import os

from oracle.routing import anchor_bits, route_frames, runs


def test_deployed_rules(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "routing_table7.json")))
    for c in g["cases"]:
        mask = route_frames(c["n_frames"], c["n_recent"], c["period"], c["n_sink"], c["all_full_until"])
        assert [f for f, m in enumerate(mask) if m] == c["full"], c["rule"]
    for kb, vb, want in g["anchor_bits"]:
        assert anchor_bits(kb, vb) == want


def test_runs_cover_the_history_in_order():
    mask = route_frames(21, 4, 16)
    r = runs(mask)
    assert r == [(0, 1, True), (1, 16, False), (16, 21, True)]
    assert sum(e - f for f, e, _ in r) == 21
    assert runs([]) == []
