"""Stored fixtures: the D3D page's packed-budget table, and the oracle's own
tiny-step outputs (written by tests/golden/make_golden.py from the oracle only;
a change here must be justified by the pages)."""
import json
import os

import numpy as np

from branch_verify_amd import synth

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_d3d_budget_table():
    with open(os.path.join(HERE, "d3d_budget.json")) as fh:
        tab = json.load(fh)
    for r in tab["rows"]:
        assert r["B"] * ((r["C"] - 1) * r["F"] + 2) == r["budget"]
    wl = synth.WORKLOADS[4]
    assert wl.B1 == (12 - 1) * 2 + 2          # one tray per covered rejection point, plus two
    assert wl.B1 * wl.N == tab["rows"][0]["budget"]


def test_tiny_step_fixture_reproduces():
    import importlib.util
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(HERE, "make_golden.py"))
    mg = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mg)
    with open(os.path.join(HERE, "tiny_step.json")) as fh:
        want = json.load(fh)
    got = mg.tiny_step()
    for k in ["parent", "state", "rows", "token", "commit_pos", "next_state", "chain", "h"]:
        assert got[k] == want[k], k
    np.testing.assert_allclose(got["lse_head"], want["lse_head"], rtol=1e-12)
    np.testing.assert_allclose(got["o_sum"], want["o_sum"], rtol=1e-9)
    np.testing.assert_allclose(got["logits_sum"], want["logits_sum"], rtol=1e-9)
