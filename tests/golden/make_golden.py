"""Writes the stored expected values under tests/golden/ by calling only the
oracle.  Run from the repository root: python tests/golden/make_golden.py"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402


def main():
    # G = [[3,0,0],[0,4,0]]: ||G||_F = 5, singular values 3 and 4 with identity
    # singular vectors, so NS5(G) = diag(g^5(0.6), g^5(0.8)) padded with a zero
    # column ("Muon Optimizer and the Distributed Implementation", section
    # "Newton-Schulz Iteration": phi acts on each singular value through
    # g(x) = a x + b x^3 + c x^5, after G <- G / ||G||_F).
    out = {
        "citation": "Muon Optimizer and the Distributed Implementation, 'Newton-Schulz Iteration': "
                    "phi(G) = U (a S + b S^3 + c S^5) V^T, coefficients (3.4445, -4.7750, 2.0315), "
                    "five steps, after Frobenius normalization",
        "G": [[3.0, 0.0, 0.0], [0.0, 4.0, 0.0]],
        "O": [[oracle.quintic_scalar(0.6), 0.0, 0.0], [0.0, oracle.quintic_scalar(0.8), 0.0]],
        "g5_of_1": oracle.quintic_scalar(1.0),
    }
    with open(os.path.join(HERE, "ns_diag_2x3.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
