"""Writes oracle_tiny.json from the float64 oracle alone (see README.md)."""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from oracle import gmm_oracle as o  # noqa: E402

X = np.array([[0.5, -1.0, 2.0], [1.5, 0.0, 1.0], [-2.0, 3.0, 0.5], [0.0, 0.25, -1.5],
              [2.5, -2.0, 0.0], [-1.0, 1.0, 1.0], [0.75, 0.5, -0.5], [3.0, -1.5, 2.5]], np.float32)
W = np.array([0.5, 0.3, 0.2], np.float32)
MU = np.array([[0.0, 0.0, 0.0], [2.0, -1.0, 1.0], [-1.0, 2.0, 0.5]], np.float32)
VAR = np.array([[1.0, 2.0, 1.5], [0.5, 1.0, 2.0], [2.0, 0.75, 1.0]], np.float32)


def main():
    Nk, S1, S2, ll = o.estep_stats(X, W, MU, VAR, method="direct")
    w1, mu1, v1 = o.mstep(Nk, S1, S2, X.shape[0], 1e-3, MU, VAR)
    off, ids, lists, _ = o.soft_assign(X, W, MU, VAR, 0.1, 2, method="direct")
    out = {"X": X.tolist(), "weights": W.tolist(), "means": MU.tolist(), "vars": VAR.tolist(),
           "var_floor": 1e-3, "threshold": 0.1, "max_extra": 2,
           "Nk": Nk.tolist(), "S1": S1.tolist(), "S2": S2.tolist(), "loglik": ll,
           "weights1": w1.tolist(), "means1": mu1.tolist(), "vars1": v1.tolist(),
           "offsets": off.tolist(), "ids": ids.tolist()}
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
