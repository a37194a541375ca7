"""Writes tests/golden/tiny_forward4.json.

The GSPN pages print no worked numerical example, so this fixture is a
regression snapshot: the seeded 'tiny' workload (N=1, C=2, 16x16, fp32,
per-channel w; full scan and chunk_len=8) and what the fp64 oracle computes
for it.  It calls only the oracle (and the seeded input generator); nothing
here comes from the GPU path.  Run from the repository root:

    python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from linear_spatial_propagation_gspn_amd.workloads import WORKLOADS, make_inputs  # noqa: E402


def main():
    wl = WORKLOADS["tiny"]
    inp = make_inputs(wl, "cpu")
    rec = {
        "about": "seeded tiny workload and its fp64 oracle output; regression snapshot "
                 "(the GSPN pages print no worked example)",
        "workload": {"n": wl.n, "c": wl.c, "h": wl.h, "w": wl.w, "seed": wl.seed},
        "x": inp["x"].flatten().tolist(),
        "logits": [z.flatten().tolist() for z in inp["logits"]],
        "lam": [l.flatten().tolist() for l in inp["lam"]],
    }
    for chunk in (0, 8):
        y = oracle.forward4(inp["x"], inp["logits"], inp["lam"], chunk=chunk)
        rec["y_chunk%d" % chunk] = [float.hex(float(v)) for v in y.flatten()]
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_forward4.json")
    with open(out, "w") as f:
        json.dump(rec, f, separators=(",", ":"))
    print("wrote", out)


if __name__ == "__main__":
    main()
