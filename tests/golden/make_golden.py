"""Writes the oracle's regression fixtures in this folder. It calls only the
oracle and the seeded input generators, never the HIP library.

    python tests/golden/make_golden.py

tiny_step.json: the whole step on the tiny workload (B=1, one query row, 4:1
GQA, 2048-token MXFP4 cache, top-k 4, seed 0), and the same with top-k 16
(every block selected, so the output is dense causal attention). These values
are the oracle's, not the pages' (the pages print no worked example); they
guard the oracle against unintended change.
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import workloads as W  # noqa: E402
from oracle import step  # noqa: E402


def tiny_case(topk):
    inp = W.make_inputs(W.WORKLOADS["tiny"].with_(topk=topk))
    r = step.decode_step_ref(inp)
    return {
        "topk": topk,
        "block_table": r["block_table"][0, 0].tolist(),
        "scores": [float(x) for x in r["scores"][0, 0]],
        "q8_first16": r["q8"][0, 0, 0, :16].tolist(),
        "O_head0": [float(x) for x in r["O"][0, 0, 0]],
        "lse": [float(x) for x in r["lse"][0, 0]],
    }


def main():
    out = {"workload": "tiny", "cases": [tiny_case(4), tiny_case(16)]}
    with open(os.path.join(HERE, "tiny_step.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
