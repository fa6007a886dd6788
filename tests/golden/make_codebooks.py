"""Write tests/golden/codebooks.json from the oracle alone.

"empirical": the exporter's Lloyd-Max procedure on RandomState(0).randn(400000),
200 iterations, quantile start, divided by sqrt(128), fp32
[OpenNeedle reference, codebook generation].  Its 2-bit entry equals the
printed CQ2 header values (checked by tests/test_oracle_codebook.py).
"gaussian": the analytic Lloyd-Max centres of N(0,1) divided by sqrt(128), fp32.

Run from the repository root:  python tests/golden/make_codebooks.py
"""
import json
import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402


def build():
    out = {"group": 128, "empirical": {}, "gaussian": {}}
    for bits in (2, 3, 4):
        L = 1 << bits
        out["empirical"][str(bits)] = [float(v) for v in oracle.lloyd_max_empirical(L)]
        g = (oracle.gaussian_lloyd_max(L) / math.sqrt(128)).astype(np.float32)
        out["gaussian"][str(bits)] = [float(v) for v in g]
    return out


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "codebooks.json")
    with open(path, "w") as f:
        json.dump(build(), f, indent=1)
        f.write("\n")
    print("wrote", path)
