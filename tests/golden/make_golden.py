"""Write the stored oracle outputs under tests/golden/.

Calls only the oracle and the seeded generator.  Run from the repository
root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402


def main():
    cfg = synth.get_config("tiny")
    res = {}
    for variant in ("base", "sharp"):
        wl = synth.make_workload(cfg, variant=variant)
        out, lse = oracle.attend(wl)
        res[variant] = {"out": [float(x) for x in out.ravel()], "lse": [float(x) for x in lse.ravel()]}
    res["about"] = ("fp64 oracle output for the tiny workload (1 head, d=64, 4 blocks x 256 tokens, "
                    "ranks 8/16/24/32, fp32, seed 0), written by tests/golden/make_golden.py")
    with open(os.path.join(ROOT, "tests", "golden", "oracle_tiny.json"), "w") as f:
        json.dump(res, f, indent=1)


if __name__ == "__main__":
    main()
