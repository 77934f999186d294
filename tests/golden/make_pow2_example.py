"""Write pow2_attention_example.json: an exact worked example of attention.

With ``scale = ln 2`` and integer Q and K, every exponential of a score is an
integer power of two, exp(S_ij) = 2 ** (q_i . k_j).  The softmax weights, the
output rows and exp(LSE) are then exact rationals, computed here with
``fractions.Fraction`` straight from the definition of scaled-dot-product
attention (softmax of the scaled scores over the allowed keys, times V).  The
causal mask is top-left: query i sees keys 0..i.

This script imports neither the oracle nor the HIP library.  Run it from the
repository root to regenerate the fixture; a test checks the stored file
against a fresh run.
"""

import json
import os
from fractions import Fraction

Q = [[1, 0, -1], [2, 1, 0], [0, -1, 1], [-1, 2, 1]]
K = [[1, 1, 0], [0, 2, -1], [-1, 0, 1], [2, -1, 1], [0, 0, 0]]
V = [[3, -1], [0, 2], [-2, 5], [1, 1], [4, -3]]


def dot(a, b):
    return sum(x * y for x, y in zip(a, b))


def example(causal):
    out_rows, r_rows = [], []
    for i, q in enumerate(Q):
        weights = []
        for j, k in enumerate(K):
            if causal and j > i:
                weights.append(Fraction(0))
            else:
                weights.append(Fraction(2) ** dot(q, k))
        total = sum(weights)
        row = [sum(w * V[j][c] for j, w in enumerate(weights)) / total for c in range(len(V[0]))]
        out_rows.append([str(x) for x in row])
        r_rows.append(str(total))
    return {"O": out_rows, "R": r_rows}


def build():
    return {
        "about": ("Exact attention example: scale = ln 2, integer Q/K/V, so exp(S_ij) = "
                  "2**(q_i.k_j). O holds exact fractions; LSE_i = ln(R_i). Causal is top-left."),
        "Q": Q, "K": K, "V": V,
        "noncausal": example(False),
        "causal": example(True),
    }


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "pow2_attention_example.json")
    with open(path, "w") as f:
        data = build()
        f.write("{\n" + ",\n".join(" %s: %s" % (json.dumps(k), json.dumps(v)) for k, v in data.items()) + "\n}\n")
    print("wrote", path)
