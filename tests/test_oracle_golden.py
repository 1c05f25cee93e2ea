"""The oracle still reproduces its committed regression fixture
(tests/golden/tiny_step.json, written by tests/golden/make_golden.py)."""
import json
import os

import numpy as np

import workloads as W
from oracle import step

GOLD = os.path.join(os.path.dirname(__file__), "golden", "tiny_step.json")


def test_tiny_step_matches_fixture():
    gold = json.load(open(GOLD))
    for case in gold["cases"]:
        inp = W.make_inputs(W.WORKLOADS["tiny"].with_(topk=case["topk"]))
        r = step.decode_step_ref(inp)
        assert r["block_table"][0, 0].tolist() == case["block_table"]
        assert r["q8"][0, 0, 0, :16].tolist() == case["q8_first16"]
        np.testing.assert_allclose(r["scores"][0, 0], case["scores"], rtol=1e-12)
        np.testing.assert_allclose(r["O"][0, 0, 0], case["O_head0"], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(r["lse"][0, 0], case["lse"], rtol=1e-12)
