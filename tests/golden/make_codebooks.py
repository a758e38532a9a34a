"""Write the oracle's Lloyd-Max codebooks for d = 128 to codebooks_d128.txt.

Calls only the CPU oracle (oracle/tq_oracle.py).  Run from the repository root:
    python tests/golden/make_codebooks.py
The 8-bit table takes about 20 s of plain Lloyd iteration.
"""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from oracle import tq_oracle as o  # noqa: E402

D = 128


def main():
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "codebooks_d128.txt")
    lines = ["# Lloyd-Max codebooks for the density (1-x^2)^((d-3)/2), d = 128.",
             "# Written by tests/golden/make_codebooks.py from oracle.tq_oracle.make_codebook.",
             "# Format: 'bits <b> iterations <n>' then one line of 2^b centroids (ascending),",
             "# then one line of 2^b - 1 boundaries, all as repr() of fp64."]
    for bits in (1, 2, 3, 4, 8):
        c, t, it = o.make_codebook(D, bits)
        lines.append(f"bits {bits} iterations {it}")
        lines.append(" ".join(repr(float(x)) for x in c))
        lines.append(" ".join(repr(float(x)) for x in t))
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
