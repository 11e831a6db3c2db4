"""Writes the expected values of the ring-simulator worked example.

Inputs are the ones printed in the simulator of the systemcraft.online course
page on agentic and multimodal distributed systems (section 8, production-grade
TypeScript simulation): 4 workers, scalar embeddings q_i = 0.5 (i+1),
k_j = 0.4 (j+1), v_j = 10 (j+1), logit s_ij = q_i k_j (head dimension 1, so the
1/sqrt(d) scale is 1).  The page prints no outputs; the expected values are
computed here by the pure-Python brute-force oracle only.

Run from the repository root:  python tests/golden/make_golden.py
"""

import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))

from oracle import brute  # noqa: E402

N = 4
q = [[[0.5 * (i + 1)]] for i in range(N)]
k = [[[0.4 * (j + 1)]] for j in range(N)]
v = [[[10.0 * (j + 1)]] for j in range(N)]
A, M, L, LSE = brute.attend(q, k, v, scale=1.0)
out = {
    "source": "systemcraft.online course page, section 8 RingAttention simulator (inputs); expected values from oracle.brute (this script)",
    "n_devices": N,
    "q": [x[0][0] for x in q],
    "k": [x[0][0] for x in k],
    "v": [x[0][0] for x in v],
    "scale": 1.0,
    "expected": {
        "A": [A[i][0][0] for i in range(N)],
        "m": [M[i][0] for i in range(N)],
        "l": [L[i][0] for i in range(N)],
        "lse": [LSE[i][0] for i in range(N)],
    },
}
path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "ring_simulator_worked_example.json")
with open(path, "w") as f:
    json.dump(out, f, indent=2)
    f.write("\n")
print(path)
