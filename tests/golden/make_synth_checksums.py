"""Write synth_checksums.json: regression checksums of the seeded workloads.

Calls only `synth` (to draw the inputs) and `oracle` (to sum them), never the
HIP library.  Run from the repository root:  python tests/golden/make_synth_checksums.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

PREFIX = 1 << 20


def main():
    out = {"prefix": PREFIX, "workloads": {}}
    for name in sorted(synth.WORKLOADS):
        x = synth.workload(name, n=PREFIX)
        out["workloads"][name] = {
            "first8": [int(v) for v in x[:8]],
            "sum": oracle.reduce(x, oracle.SUM),
            "max": oracle.reduce(x, oracle.MAX),
            "min": oracle.reduce(x, oracle.MIN),
        }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "synth_checksums.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
