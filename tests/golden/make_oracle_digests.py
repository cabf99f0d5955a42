"""Write oracle_workload1.json: digests of the oracle's outputs on workload 1.

Calls only the oracle and the seeded generators.  The stored digests let a
later change to the oracle's arithmetic show up as a failing test, which must
then name the passage (or reading) that justifies the change.
Run:  python tests/golden/make_oracle_digests.py
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle as O  # noqa: E402
from weight_only_quantization_pack_amd import workloads as WL  # noqa: E402


def digest(a) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def compute():
    wl = WL.workload(1)
    W, X = wl.weights(), wl.calibration()
    s_x = O.act_stat(X)
    s = O.candidate_scale(s_x, 0.5)
    out = {"s_x": digest(s_x), "s_alpha_0.5": digest(s)}
    for bits in (4, 3):
        q, d, z = O.quantize(W, s, bits)
        out[f"int{bits}"] = {"qweight": digest(O.pack(q, bits)), "scales": digest(d),
                             "zeros": digest(z)}
        _, losses, best = O.search_scale(W, X, wl.alphas + [0.0, 1.0], bits)
        out[f"int{bits}"]["search_best"] = best
        out[f"int{bits}"]["search_losses"] = [float(v) for v in losses]
    return out


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_workload1.json")
    json.dump(compute(), open(path, "w"), indent=1)
    print("wrote", path)
