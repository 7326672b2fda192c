"""Write workload_digests.json: SHA-256 of every synthetic workload's input arrays.

Calls only the seeded input generator (``workloads``), never the HIP library. The digests pin the
generator's bytes so that both the oracle and the GPU path are known to consume identical inputs
(and a numpy change in the draws would show up as a failing test, not as a silent parity drift).
Run from the repository root: ``python tests/golden/make_digests.py``.
"""
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from workloads import WORKLOADS, make_workload  # noqa: E402

out = {}
for i, name in WORKLOADS.items():
    wl = make_workload(i)
    out[str(i)] = {"name": name, "B": wl.B, "V": wl.V, "dtype": wl.dtype, "R": wl.R, "W": wl.W,
                   "sha256": wl.digest()}
    print(i, name, out[str(i)]["sha256"])
path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "workload_digests.json")
json.dump(out, open(path, "w"), indent=2)
