"""Write tests/golden/tiny_f32_oracle.json from the float64 oracle.

The fixture freezes the oracle's output on the seeded tiny_f32 workload
(B=1, H=1, T=256, d_k=d_v=16) so that any later change to the oracle's
arithmetic shows up as a failing test and has to be justified when the file is
regenerated.  It calls only oracle/ and kla_inputs/.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import kla_inputs as KI  # noqa: E402
from oracle import kla_forward_f64  # noqa: E402

ROWS = [0, 1, 2, 15, 16, 17, 100, 200, 254, 255]


def compute():
    x = KI.make_forward_inputs("tiny_f32")
    y, lT, MT, path = kla_forward_f64(x["q"], x["k"], x["v"], x["log_decay"], x["proc_noise"],
                                      x["val_prec"], x["lambda0"], x["M0"], return_lambda_path=True)
    return {
        "workload": "tiny_f32", "seed": x["seed"], "rows": ROWS,
        "y_rows": [[float(u) for u in y[0, 0, t]] for t in ROWS],
        "lambda_rows": [[float(u) for u in path[0, 0, t]] for t in ROWS],
        "lambda_T": [float(u) for u in lT[0, 0]],
        "M_T_diag": [float(MT[0, 0, i, i]) for i in range(16)],
    }


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_f32_oracle.json")
    with open(out, "w") as f:
        json.dump(compute(), f, indent=1)
    print("wrote", out)
