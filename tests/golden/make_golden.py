"""Writes oracle_tiny_trajectory.json: the oracle's float32 trajectory on a
tiny seeded layer, kept as a regression anchor for the oracle itself.

Calls only the seeded generators and the oracle. Run from the repo root:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from synth import DenseCase, dense_inputs, dense_state  # noqa: E402

CASE = DenseCase("golden_tiny", T=40, d_in=16, d_out=8, seed_base=9000, steps=3)


def hexbits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).ravel().tolist()


def trajectory():
    W, m, v = dense_state(CASE)
    Ws, bs = W.copy(), np.zeros_like(W)
    out = {"case": CASE.__dict__, "adamw": [], "sgdm": []}
    for t in range(1, CASE.steps + 1):
        X, dY = dense_inputs(CASE, t)
        g = oracle.wgrad(X, dY)
        W, m, v = oracle.adamw_step(W, m, v, g, t, lr=CASE.lr, beta1=CASE.beta1,
                                    beta2=CASE.beta2, eps=CASE.eps,
                                    weight_decay=CASE.weight_decay)
        Ws, bs = oracle.sgdm_step(Ws, bs, g, lr=CASE.lr, momentum=CASE.momentum,
                                  weight_decay=CASE.weight_decay)
        out["adamw"].append({"g": hexbits(g), "W": hexbits(W), "m": hexbits(m), "v": hexbits(v)})
        out["sgdm"].append({"W": hexbits(Ws), "b": hexbits(bs)})
    return out


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny_trajectory.json")
    with open(path, "w") as f:
        json.dump(trajectory(), f, separators=(",", ":"))
    print("wrote", path)
