"""Write input_fingerprints.json: SHA-256 of each workload's generated inputs.

Uses only the seeded generator (no oracle, no GPU).  Run from the repository
root: python tests/golden/make_fingerprints.py
"""
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import skinny_inputs as si  # noqa: E402

out = {}
for cid in (1, 4):
    out[str(cid)] = {"weight0": si.fingerprint(si.weight(cid)),
                     "x": si.fingerprint(si.activations(cid))}
path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "input_fingerprints.json")
with open(path, "w") as f:
    json.dump(out, f, indent=1, sort_keys=True)
    f.write("\n")
print(path)
