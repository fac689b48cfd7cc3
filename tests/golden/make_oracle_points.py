"""Writes oracle_points.txt: the fp64 oracle's act and act' at fixed points.

Calls only the oracle package.  Run from the repository root:
    python tests/golden/make_oracle_points.py
The file is a regression fixture (it detects unintended changes to the
oracle's arithmetic); the oracle's correctness is established by the pins.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402

POINTS = [0.0, 1.0, -1.0, 2.0, -2.0, 0.5, -0.5, 3.0, -3.0, 5.0, -5.0, 10.0, -10.0,
          40.0, -40.0, -80.0, -1.2784645427610738, -0.7517915246935645,
          -0.7524614220710162, 1e-6, -1e-6, 13.5, -13.5, 88.75, -88.75]


def main():
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_points.txt")
    with open(out, "w") as f:
        f.write("# kind function x value  (hex floats; written by make_oracle_points.py)\n")
        for kind in ("silu", "gelu_erf", "gelu_tanh", "relu"):
            for fn, call in (("act", oracle.act1), ("dact", oracle.dact1)):
                for x in POINTS:
                    f.write(f"{kind} {fn} {float(x).hex()} {call(kind, x).hex()}\n")
    print("wrote", out)


if __name__ == "__main__":
    main()
