"""Writes tests/golden/oracle_regression.json by calling only the oracle.

This is a regression fixture, not a pin: it records the oracle's own output on a small
closed-form input (no random numbers), so a later change to the oracle's arithmetic
shows up as a diff. The oracle is pinned to mathematics in tests/test_oracle_pins.py.
Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import nystrom_forward  # noqa: E402


def closed_form_inputs(n=24, d=4, H=2, W=5):
    t = np.arange(n)[:, None]
    c = np.arange(d)[None, :]
    q = np.stack([np.sin(0.37 * t + 0.11 * c + h) for h in range(H)])[None]
    k = np.stack([np.cos(0.23 * t - 0.17 * c + 0.5 * h) for h in range(H)])[None]
    v = np.stack([np.sin(0.05 * t * (c + 1) + h) for h in range(H)])[None]
    w = np.stack([np.linspace(-0.3, 0.4, W) * (h + 1) for h in range(H)])
    return q, k, v, w


def main():
    q, k, v, w = closed_form_inputs()
    m, iters = 6, 6
    out, attn = nystrom_forward(q, k, v, w, m, iters)
    payload = {
        "about": "oracle regression fixture; inputs are closed_form_inputs() in make_golden.py",
        "m": m, "iters": iters, "shape": list(out.shape),
        "out": [float(f"{x:.17g}") for x in out.ravel()],
        "attn": [float(f"{x:.17g}") for x in attn.ravel()],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_regression.json")
    with open(path, "w") as fh:
        json.dump(payload, fh, indent=0)
    print("wrote", path)


if __name__ == "__main__":
    main()
