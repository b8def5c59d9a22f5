"""Writes tests/golden/tiny_attention.json from the oracle only.

The pages print no worked numeric example with fixed inputs, so this fixture
is a regression record of the oracle on a tiny hand-written case (integer
inputs, so anyone can recompute it by hand or with another tool). Run from the
repository root: ``python tests/golden/make_golden.py``.
"""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from oracle.attention import attention  # noqa: E402

Q = [[1, 0, 0, 1], [0, 2, 1, 0], [1, 1, 1, 1]]
K = [[1, 1, 0, 0], [0, 0, 2, 1], [-1, 0, 1, 0]]
V = [[1, 2, 3, 4], [0, -1, 0, 1], [2, 0, -2, 0]]


def main():
    q = np.array(Q, float)[None, :, None, :]
    k = np.array(K, float)[None, :, None, :]
    v = np.array(V, float)[None, :, None, :]
    out = {"alpha": 0.5, "Q": Q, "K": K, "V": V}
    for causal in (False, True):
        o, lse = attention(q, k, v, 0.5, causal)
        out["causal" if causal else "full"] = {"O": o[0, :, 0].tolist(), "LSE": lse[0, 0].tolist()}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_attention.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
