"""Write tiny_oracle.json: a small case and the oracle's outputs for it.

Calls only ``oracle/`` (and the seeded input generator).  The pages print no
worked numeric example, so this fixture is a regression guard on the oracle
itself: any change to its arithmetic changes these numbers, and such a change
must name the passage (or the reading of it) that justifies it.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from rope_head_mixing_amd import synthetic  # noqa: E402

SQ, NH, NOPE, PE, THETA = 4, 3, 8, 8, 10000.0
POSITIONS = [0, 1, 100, 32767]


def main():
    c = synthetic.case(SQ, NH, NOPE, PE, seed=4242)
    O, W, dY = c.O(), c.W(), c.dY()
    Y = oracle.fwd(O, W, POSITIONS, THETA, NOPE, PE, nthreads=1)
    dO = oracle.bwd_dx(dY, W, POSITIONS, THETA, NOPE, PE, nthreads=1)
    dW = oracle.bwd_dw(dY, O, POSITIONS, THETA, NOPE, PE, nthreads=1)
    doc = {
        "what": "oracle outputs for a tiny case (regression guard; not values from the pages)",
        "source": "PaddleFleet PR #1772, PR body item 1 and description part 一: "
                  "Y = W . inv_rope(O); dO = rope(W^T dY); dW = sum dY * inv_rope(O)",
        "shape": {"sq": SQ, "nh": NH, "nope": NOPE, "pe": PE, "theta": THETA},
        "positions": POSITIONS,
        "O_bf16_hex": [f"{v:04x}" for v in O.reshape(-1).tolist()],
        "W_bf16_hex": [f"{v:04x}" for v in W.reshape(-1).tolist()],
        "dY_bf16_hex": [f"{v:04x}" for v in dY.reshape(-1).tolist()],
        "Y": [repr(v) for v in Y.reshape(-1).tolist()],
        "dO": [repr(v) for v in dO.reshape(-1).tolist()],
        "dW": [repr(v) for v in dW.reshape(-1).tolist()],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=0)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
