"""Plant plausible mistakes in copies of the W4A8 oracle and check that its pins catch each.

Every mutant is the W4A8 oracle's own source with one edit, executed into a fresh module
(within the oracle package, so that its relative imports resolve) on the CPU.
"""
import os
import types

import pytest

import oracle_pins_w4a8

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "w4a8_oracle.py")

MUTANTS = [
    ("exponent bias 8 (the FNUZ variant) in decode",
     "np.exp2(e.astype(np.float64) - E4M3_BIAS)", "np.exp2(e.astype(np.float64) - E4M3_BIAS - 1)"),
    ("largest finite value 240",
     "E4M3_MAX = 448.0", "E4M3_MAX = 240.0"),
    ("mantissa step 1/16",
     "normal = (1.0 + m / 8.0)", "normal = (1.0 + m / 16.0)"),
    ("subnormals one binade too low",
     "subnormal = (m / 8.0) * np.exp2(1.0 - E4M3_BIAS)", "subnormal = (m / 8.0) * np.exp2(0.0 - E4M3_BIAS)"),
    ("ties always up",
     "((d_hi == d_lo) & (hi % 2 == 0))", "(d_hi == d_lo)"),
    ("ties to odd",
     "((d_hi == d_lo) & (hi % 2 == 0))", "((d_hi == d_lo) & (hi % 2 == 1))"),
    ("sign dropped by encode",
     "return code | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)", "return code"),
    ("one scale for the whole tensor",
     "amax = np.abs(x32).max(axis=1)", "amax = np.full(x32.shape[0], np.abs(x32).max())"),
    ("activations multiplied by the scale instead of divided",
     "scaled = (x32 / sx[:, None]).astype(np.float32)", "scaled = (x32 * sx[:, None]).astype(np.float32)"),
    ("zero row scale 0",
     "np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0))", "amax / np.float32(E4M3_MAX)"),
    ("row scale left out of the product",
     "return y * np.asarray(sx, dtype=np.float64)[:, None]", "return y"),
    ("weight values without the zero point",
     "return codes.astype(np.float64) - z", "return codes.astype(np.float64)"),
    ("weight values add the zero point",
     "return codes.astype(np.float64) - z", "return codes.astype(np.float64) + z"),
    ("weight values rounded to E4M3 (8-bit weight operand q - z)",
     "return codes.astype(np.float64) - z", "return e4m3_decode(e4m3_encode(codes.astype(np.float64) - z))"),
    ("zero point clamped to the 4-bit code range",
     "return codes.astype(np.float64) - z", "return codes.astype(np.float64) - np.clip(z, 0, 15)"),
    ("block sums over 64 rows",
     "BLOCK = 128               # R22", "BLOCK = 64                # R22"),
    ("block sums of magnitudes",
     "return a.reshape(M, K // BLOCK, BLOCK).sum(axis=2).T", "return np.abs(a).reshape(M, K // BLOCK, BLOCK).sum(axis=2).T"),
    ("block sums row-major [M, K/128]",
     "return a.reshape(M, K // BLOCK, BLOCK).sum(axis=2).T", "return a.reshape(M, K // BLOCK, BLOCK).sum(axis=2)"),
    ("first group's scale for every group",
     "y += (a[:, rows] @ w[rows, :]) * s[g][None, :]", "y += (a[:, rows] @ w[rows, :]) * s[0][None, :]"),
    ("last group dropped",
     "for g in range(K // group_size):", "for g in range(K // group_size - 1):"),
]


def _load_mutant(old, new):
    src = open(SRC_PATH).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new)
    mod = types.ModuleType("oracle.w4a8_mutant")
    mod.__package__ = "oracle"
    exec(compile(src, "oracle_w4a8_mutant", "exec"), mod.__dict__)
    return mod


def test_mutation_anchors_present():
    src = open(SRC_PATH).read()
    for name, old, _ in MUTANTS:
        assert src.count(old) >= 1, name


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    mod = _load_mutant(old, new)
    caught = []
    for pin in oracle_pins_w4a8.ALL_PINS:
        try:
            pin(mod)
        except Exception:            # a wrong value or a crash both expose the mutant
            caught.append(pin.__name__)
    assert caught, f"no pin caught the mutant: {name}"
