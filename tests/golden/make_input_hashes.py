"""Writes tests/golden/input_hashes.json: SHA-256 of the seeded workload tensors.

Run from the repository root: python tests/golden/make_input_hashes.py
It calls only the seeded generator; the hashes freeze the generator's output so that a change in
it (seeding, scaling, rounding, outlier columns) is caught.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from sparse_rank_linear_prune24_amd import inputs  # noqa: E402

CASES = [("C1", 0), ("C2", 0), ("C3", 0)]


def main():
    out = {}
    for cfg, layer in CASES:
        L = inputs.make_layer(cfg, layer)
        out[f"{cfg}/{layer}"] = inputs.layer_hashes(L)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "input_hashes.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
