"""Writes c0_oracle_step.json: the oracle's full draft step on the tiny fp32
workload (V=8192, d=256, 64 contiguous clusters of 128, cluster budgets
8, 6, 4, 4, seeded inputs, instance 0).

The pages print no worked example for any step, so this file is a regression
pin of the oracle only: it records what the oracle computed when its pins
(tests/test_oracle.py) passed.  It calls nothing but oracle/ and the seeded
input generator.  Run from the repository root:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from oracle import pipeline  # noqa: E402
from dynamic_vocabulary_draft_amd import synthetic as syn  # noqa: E402


def c0_summary():
    wl = syn.make_workload(0)
    r = pipeline.run_step(wl)
    return {
        "workload": wl.cfg.name,
        "selected": [s[0, : n[0]].tolist() for s, n in zip(r["sel"], r["n_sel"])],
        "sl_len": [int(x[0]) for x in r["sl_len"]],
        "sl_off": r["sl_off"].tolist(),
        "draft": r["token"].reshape(-1).tolist(),
        "n_acc": r["n_acc"].tolist(),
        "out": r["out"].tolist(),
        "logits_first8": [float(np.float32(x)) for x in r["logits"][:8]],
        "scores_row0_first8": [float(x) for x in r["scores"][0][0, :8]],
    }


if __name__ == "__main__":
    oracle.build(force=False)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c0_oracle_step.json")
    with open(path, "w") as f:
        json.dump(c0_summary(), f, indent=1)
    print("wrote", path)
