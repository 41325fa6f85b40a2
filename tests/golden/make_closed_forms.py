"""Writes the closed-form fixtures in this folder from their identities.

lse_closed_form.txt: a constant row x_v = c of length V has
log sum_v exp(x_v) = c + log V. Only the math module is used.
Run from the repository root: python tests/golden/make_closed_forms.py
"""
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def main():
    lines = ["# Closed form: a constant row x_v = c of length V has log sum_v exp(c) = c + log V.",
             "# Values written out from that identity (independent of any implementation).",
             "# c  V  lse"]
    for c, V in [(0.0, 1), (0.0, 151936), (1.75, 5000), (-3.5, 1024), (12.0, 151937), (-0.0, 7)]:
        lines.append(f"{c!r} {V} {c + math.log(V):.15f}")
    with open(os.path.join(HERE, "lse_closed_form.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
