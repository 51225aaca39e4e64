"""Writes tests/golden/tiny_exact.json: the exact rational result of a
hand-sized KDA problem (T=5 tokens, K=3 key channels, V=2 value channels,
one head), computed only with ``oracle.exact`` (fractions, no rounding).

Run from the repository root:  python tests/golden/make_tiny_exact.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle.exact import rational_problem, transition_form  # noqa: E402


def main():
    q, k, v, alpha, beta, S0 = rational_problem(2024, 5, 3, 2)
    o, S = transition_form(q, k, v, alpha, beta, S0)
    s = lambda m: [[str(x) for x in row] for row in m]
    fx = {
        "about": "exact rationals from oracle.exact.transition_form; g = ln(alpha)",
        "q": s(q), "k": s(k), "v": s(v), "alpha": s(alpha), "beta": [str(x) for x in beta], "S0": s(S0),
        "o": s(o), "S_final": s(S),
    }
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_exact.json")
    with open(out, "w") as f:
        json.dump(fx, f, indent=1)
    print("wrote", out)


if __name__ == "__main__":
    main()
