"""Write tests/golden/oracle_small.json from the oracle alone.

The pages print no worked numeric example, so the only stored expected values are these,
written by this script, which calls nothing but oracle/ and the seeded input generator.
A change to this file means the oracle's arithmetic changed, which needs a reason.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402

M, K, N = 3, 256, 12


def build():
    W = synth.weight(K, N, wid=0, layer=0)
    x = synth.activations(M, K, wid=0)
    qw, s, z = oracle.quantize_pack(W)
    y = oracle.matmul(x, qw, s, z)
    return {
        "about": "oracle output on synth.weight(256, 12) / synth.activations(3, 256), group 128",
        "M": M, "K": K, "N": N, "group_size": 128,
        "qweight_u32_hex": [[f"{v:08x}" for v in row] for row in qw.view(np.uint32).tolist()],
        "scales_f16_hex": [[f"{v:04x}" for v in row] for row in s.view(np.uint16).tolist()],
        "zeros_f16": z.astype(float).tolist(),
        "y_f64_hex": [[float(v).hex() for v in row] for row in y.tolist()],
    }


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small.json")
    with open(out, "w") as f:
        json.dump(build(), f, indent=1)
        f.write("\n")
    print("wrote", out)
