"""Writes tests/golden/c1_oracle.json from the float64 oracle only (no GPU code involved).

Run from the repository root:  python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402
from oracle import kronq as kq  # noqa: E402


def main():
    sp = synth.CONFIGS["C1"]
    d = synth.layer_inputs(sp)
    r = kq.quantize_layer(synth.widen(d["X"], sp.x_dtype), synth.widen(d["W"], sp.w_dtype),
                          d["HG"].astype(np.float64), sp.hg_form, d["s"], d["t"], sp.bits, sp.group,
                          sp.block, sp.damp)
    out = {"workload": sp.name, "note": "oracle outputs of the 256x256 W4 per-row workload",
           "words_sha256": hashlib.sha256(r["words"].tobytes()).hexdigest(),
           "loss": r["loss"], "loss_rot": r["loss_rot"], "score": r["score"], "lambda": r["lam"],
           "min_tie_distance": float(r["delta"].min())}
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "c1_oracle.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(out)


if __name__ == "__main__":
    main()
