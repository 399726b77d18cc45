"""Writes workload_sha256.json: the SHA-256 of every array the seeded
generators draw for the tiny fp32 forward and the tiny skewed training
workloads, with the numpy version that drew them.

Run from the repository root: python tests/golden/make_workload_sha256.py
The arrays are inputs (drawn by static_token_routed_id_amd/workloads.py,
which holds no arithmetic of the layer); nothing here is an expected output.
"""
import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from static_token_routed_id_amd import workloads as wl  # noqa: E402

NAMES = ("tiny_fp32", "train_skew_bf16")
FIELDS = ("ids", "offsets", "x", "K", "V", "W_up", "gamma", "beta", "W_mix",
          "dy")


def digests(name):
    w = wl.make(name)
    out = {}
    for f in FIELDS:
        a = getattr(w, f)
        if a is None:
            continue
        a = np.ascontiguousarray(a)
        h = hashlib.sha256()
        h.update(f"{a.dtype.str}{a.shape}".encode())
        h.update(a.tobytes())
        out[f] = h.hexdigest()
    return out


def main():
    rec = {"numpy": np.__version__,
           "workloads": {n: digests(n) for n in NAMES}}
    with open(os.path.join(HERE, "workload_sha256.json"), "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
