"""The oracle still reproduces the frozen small case (tests/golden/oracle_small.json)."""
import json
import os

import numpy as np

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "oracle_small.json")


def test_oracle_matches_frozen_small_case():
    g = json.load(open(GOLDEN))
    W = synth.weight(g["K"], g["N"], wid=0, layer=0)
    x = synth.activations(g["M"], g["K"], wid=0)
    qw, s, z = oracle.quantize_pack(W, g["group_size"])
    assert [[f"{v:08x}" for v in r] for r in qw.view(np.uint32).tolist()] == g["qweight_u32_hex"]
    assert [[f"{v:04x}" for v in r] for r in s.view(np.uint16).tolist()] == g["scales_f16_hex"]
    assert z.astype(float).tolist() == g["zeros_f16"]
    y = oracle.matmul(x, qw, s, z, g["group_size"])
    want = np.array([[float.fromhex(v) for v in r] for r in g["y_f64_hex"]])
    # the fp64 sum's last bits depend on the BLAS summation order; the products are exact
    assert np.allclose(y, want, rtol=0, atol=g["K"] * 2.0 ** -50 * np.abs(want).max())
