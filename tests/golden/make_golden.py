"""Write tests/golden/swiglu_small.json from the oracle alone.

The inputs are chosen by hand to hit the method's special points: g = 0
(silu = 0, silu' = 1/2), the minimiser g0 = -1 - W(1/e) where silu' = 0,
deep saturation on both sides (|g| = 30, 100), exactly representable small
values, and zero up / zero dy. Expected values are the oracle's float64
results (as hex floats) and their one-step nearest-even bf16 roundings.

Run from the repository root: python tests/golden/make_golden.py
Regenerate only when a change to the oracle's arithmetic is justified by the
definitions it follows; the test that reads this file pins the oracle against
accidental change.
"""

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402

G = [0.0, 1.0, -1.0, 0.5, oracle.G0, -30.0, 30.0, -100.0]
U = [1.0, 2.0, -0.75, 0.0, 1.5, -1.0, 0.25, 3.0]
DY = [[1.0, 0.5, -2.0, 1.0, 1.0, 1.0, -1.0, 0.0],
      [0.25, 1.0, 1.0, -1.0, 2.0, 0.5, 1.0, 1.0]]


def main():
    x = np.array([G + U, U[::-1] + G[::-1]], dtype=np.float64)     # 2 rows, n = 8
    dy = np.array(DY, dtype=np.float64)
    y = oracle.oracle_fwd(x)
    dx = oracle.oracle_bwd(x, dy)
    hx = lambda a: [[float(v).hex() for v in row] for row in a]  # noqa: E731
    out = {
        "source": "tests/golden/make_golden.py (oracle only)",
        "layout": "x rows are [gate(0..n) | up(n..2n)], n = 8; dx rows are [dgate | dup]",
        "x": hx(x), "dy": hx(dy), "y": hx(y), "dx": hx(dx),
        "y_bf16_bits": oracle.round_f64_to_bf16_bits(y).tolist(),
        "dx_bf16_bits": oracle.round_f64_to_bf16_bits(dx).tolist(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "swiglu_small.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
