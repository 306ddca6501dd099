"""Writes int8_calibration.json: the activation scale and zero point of the
inputs of the pair MLP's layers 2, 3, 4 for the seed-0 workloads, from the
ranges of the float64 oracle MLP over their real pairs (S = (max - min) /
255, Z = -128 - rint(min / S)).  Calls only the oracle; the int8 tests and
bench.py read the file.  Run from the repository root:
    python tests/golden/make_int8_calibration.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from pair_interaction_particle_amd import synth  # noqa: E402

out = {}
for name in ("kernel", "large_bf16"):
    d = synth.make_workload(name)
    r = oracle.pair_mlp_ranges(d["p4"], d["mask"], d["mlp"])
    S, Z = oracle.int8_calibration(r)
    out[name] = {"ranges": r.tolist(), "act_scale": [float(x) for x in S],
                 "act_zero": [int(x) for x in Z]}
path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "int8_calibration.json")
with open(path, "w") as f:
    json.dump(out, f, indent=1)
print(path)
