"""Writes oracle_regression.json: hashes of the CPU oracle's state after a
few steps of a small seeded case.  Calls only the oracle (inputs are drawn
here with numpy's default generator).  The pages print no worked example with
numbers, so this file guards the oracle against unintended change rather than
pinning it; a change to the oracle's arithmetic that alters it must name, in
its commit message, the passage that justifies it.

Run:  python tests/golden/make_golden.py
"""

import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import Hyper, OracleOptimizer  # noqa: E402

CASE = {"n_p": 5000, "P": 3, "K": 2, "k": 250, "steps": 4, "seed": 1234,
        "beta1": 0.9, "beta2": 0.95, "eps": 1e-8, "weight_decay": 0.01, "lr": 1e-3}


def run(case):
    rng = np.random.default_rng(case["seed"])
    n = case["n_p"] * case["P"]
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    hp = Hyper.make(case["beta1"], case["beta2"], case["eps"], case["weight_decay"], case["lr"])
    opt = OracleOptimizer(w0, case["P"], case["K"], case["k"], hp)
    for _ in range(case["steps"]):
        g = (rng.standard_normal((case["K"], n)) * 1e-3).astype(np.float32)
        opt.step(g)
    out = {}
    for name in ("w", "m", "v", "e"):
        out[name] = hashlib.sha256(np.ascontiguousarray(opt.gather(name)).tobytes()).hexdigest()
    out["mask"] = hashlib.sha256(opt.mask_global_idx().astype(np.int64).tobytes()).hexdigest()
    return out


if __name__ == "__main__":
    doc = {"case": CASE, "sha256": run(CASE),
           "note": "regression fixture written by make_golden.py from the CPU oracle"}
    with open(os.path.join(HERE, "oracle_regression.json"), "w") as f:
        json.dump(doc, f, indent=1)
    print(json.dumps(doc["sha256"], indent=1))
