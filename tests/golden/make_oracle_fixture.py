"""Write oracle_small_case.json from the oracle alone (regression lock)."""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle.mcs_oracle import anchor_step, reuse_step  # noqa: E402


def small_case():
    """Dyadic inputs (multiples of 1/8 in [-2, 2)) from an integer generator."""
    rng = np.random.Generator(np.random.PCG64(20261203))
    nq, nk, d = 150, 150, 8
    Q = rng.integers(-16, 16, (nq, d)) / 8.0
    K = rng.integers(-16, 16, (nk, d)) / 8.0
    V = rng.integers(-16, 16, (nk, d)) / 8.0
    Q2 = Q + rng.integers(-1, 2, (nq, d)) / 8.0
    return dict(Q=Q, K=K, V=V, Q2=Q2, G=64, k=20, scale=0.5, causal_block=50, q_offset=0, iters=32)


def compute(case):
    a = anchor_step(case["Q"], case["K"], case["V"], case["G"], case["k"], case["scale"],
                    case["causal_block"], case["q_offset"], case["iters"])
    O2 = reuse_step(case["Q2"], case["K"], case["V"], a["perm"], a["idx"], a["R"], case["G"],
                    case["scale"], case["causal_block"], case["q_offset"])
    return {"perm": a["perm"].tolist(), "idx": a["idx"].tolist(),
            "O_full": a["O_full"].tolist(), "R": a["R"].tolist(), "O_reuse": O2.tolist()}


if __name__ == "__main__":
    out = compute(small_case())
    with open(os.path.join(HERE, "oracle_small_case.json"), "w") as f:
        json.dump(out, f)
    print("wrote oracle_small_case.json")
