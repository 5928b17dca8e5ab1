"""Plant plausible mistakes in copies of the oracle and check that the pins catch each.

Every mutant is the oracle's own source with one edit, executed into a fresh module on
the CPU. A mutant that passes every pin would mean the pins cannot tell that mistake
from the method, so the test fails.
"""
import os
import types

import pytest

import oracle_pins

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "w4a16_oracle.py")

MUTANTS = [
    # packing / unpacking
    ("nibble order reversed in pack",
     "codes[k::NIBBLES_PER_WORD, :].astype(np.uint32) << np.uint32(4 * p)",
     "codes[k::NIBBLES_PER_WORD, :].astype(np.uint32) << np.uint32(4 * (7 - p))"),
    ("nibble order reversed in both pack and unpack",
     "np.uint32(4 * p)", "np.uint32(4 * (7 - p))"),
    ("K split into 8 planes instead of 8 consecutive rows (pack and unpack)",
     [("words |= codes[k::NIBBLES_PER_WORD, :]", "words |= codes[k * (K // 8):(k + 1) * (K // 8), :]"),
      ("codes[k::NIBBLES_PER_WORD, :] = (words", "codes[k * P:(k + 1) * P, :] = (words")], None),
    ("interleaved map inverted (the K-offset -> nibble map used as nibble -> K offset)",
     '"interleaved": (0, 2, 4, 6, 1, 3, 5, 7)', '"interleaved": (0, 4, 1, 5, 2, 6, 3, 7)'),
    ("matmul unpacks every layout as linear",
     "codes = unpack(qweight, layout)", "codes = unpack(qweight)"),
    ("unpack mask 0x7",
     "& np.uint32(0xF)", "& np.uint32(0x7)"),
    # quantiser
    ("floor instead of round for codes",
     "q = np.rint(Wg / s[:, None, :]) + z[:, None, :]",
     "q = np.floor(Wg / s[:, None, :]) + z[:, None, :]"),
    ("zero point with the wrong sign",
     "z = np.rint(-mn / s)", "z = np.rint(mn / s)"),
    ("scale over 16 levels",
     "s32 = rng / np.float32(QMAX)", "s32 = rng / np.float32(16)"),
    ("codes computed with the unrounded fp32 scale",
     "q = np.rint(Wg / s[:, None, :]) + z[:, None, :]",
     "q = np.rint(Wg / s32[:, None, :]) + z[:, None, :]"),
    ("zero computed with the unrounded fp32 scale",
     "z = np.rint(-mn / s)", "z = np.rint(-mn / s32)"),
    ("no upper clamp",
     "q = np.clip(q, 0, QMAX)", "q = np.clip(q, 0, 16)"),
    ("groups interleaved along K (k mod G) instead of contiguous",
     "Wg = W.reshape(G, group_size, N)",
     "Wg = W.reshape(group_size, G, N).transpose(1, 0, 2)"),
    ("codes rounded after adding the zero: rne(w/s + z)",
     "q = np.rint(Wg / s[:, None, :]) + z[:, None, :]",
     "q = np.rint(Wg / s[:, None, :] + z[:, None, :])"),
    ("codes rounded half away from zero",
     "q = np.rint(Wg / s[:, None, :]) + z[:, None, :]",
     "t = Wg / s[:, None, :]; q = np.trunc(t + np.copysign(np.float32(0.5), t)) + z[:, None, :]"),
    ("zero point rounded half up",
     "z = np.rint(-mn / s)", "z = np.floor(-mn / s + np.float32(0.5))"),
    ("zero point rounded half down",
     "z = np.rint(-mn / s)", "z = np.ceil(-mn / s - np.float32(0.5))"),
    ("codes from w times a rounded reciprocal of the scale",
     "q = np.rint(Wg / s[:, None, :]) + z[:, None, :]",
     "q = np.rint(Wg * (np.float32(1) / s)[:, None, :]) + z[:, None, :]"),
    ("symmetric codes from w times a rounded reciprocal of the scale",
     "q = np.rint(Wg / s[:, None, :]) + np.float32(SYM_ZERO)",
     "q = np.rint(Wg * (np.float32(1) / s)[:, None, :]) + np.float32(SYM_ZERO)"),
    ("range from max only",
     "rng = mx - mn", "rng = mx - np.float32(0)"),
    # dequant
    ("dequant adds the zero",
     "(codes.astype(np.float32) - z) * s", "(codes.astype(np.float32) + z) * s"),
    ("dequant forgets to scale the zero",
     "(codes.astype(np.float32) - z) * s", "codes.astype(np.float32) * s - z"),
    ("dequant drops the zero",
     "(codes.astype(np.float32) - z) * s", "codes.astype(np.float32) * s"),
    ("group broadcast tiled instead of repeated",
     "s = np.repeat(np.asarray(scales).astype(np.float32), group_size, axis=0)",
     "s = np.tile(np.asarray(scales).astype(np.float32), (group_size, 1))"),
    ("fp16 dequant rounds half away from zero",
     "return dequant(codes, scales, zeros, group_size).astype(np.float16)",
     "d = dequant(codes, scales, zeros, group_size).astype(np.float64); "
     "return (np.sign(d) * np.floor(np.abs(d) * 2.0 ** 9 + 0.5) / 2.0 ** 9).astype(np.float16)"),
    # group sizes other than 128
    ("dequant broadcasts every group over 128 rows whatever the group size",
     [("s = np.repeat(np.asarray(scales).astype(np.float32), group_size, axis=0)",
       "s = np.repeat(np.asarray(scales).astype(np.float32), GROUP_SIZE, axis=0)[:K]"),
      ("z = np.repeat(np.asarray(zeros).astype(np.float32), group_size, axis=0)",
       "z = np.repeat(np.asarray(zeros).astype(np.float32), GROUP_SIZE, axis=0)[:K]")], None),
    ("quantiser groups 128 rows whatever the group size",
     "    G = K // group_size\n    Wg = W.reshape(G, group_size, N)                      # Wg",
     "    G = K // GROUP_SIZE\n    Wg = W.reshape(G, GROUP_SIZE, N)                      # Wg"),
    # symmetric mode
    ("symmetric scale over 8 levels",
     "s32 = amax / np.float32(SYM_QPOS)", "s32 = amax / np.float32(8)"),
    ("symmetric zero point 7",
     "q = np.rint(Wg / s[:, None, :]) + np.float32(SYM_ZERO)",
     "q = np.rint(Wg / s[:, None, :]) + np.float32(7)"),
    ("symmetric scale from the maximum instead of the largest magnitude",
     "amax = np.abs(Wg).max(axis=1)", "amax = Wg.max(axis=1)"),
    ("symmetric codes from floor",
     "q = np.rint(Wg / s[:, None, :]) + np.float32(SYM_ZERO)",
     "q = np.floor(Wg / s[:, None, :]) + np.float32(SYM_ZERO)"),
    ("symmetric mode falls back to the asymmetric quantiser",
     "        return _quantize_symmetric(W, group_size)", "        pass"),
    # matmul
    ("matmul accumulates in fp32",
     "w = dequant(codes, scales, zeros, group_size).astype(np.float64)\n    return x.astype(np.float64) @ w",
     "w = dequant(codes, scales, zeros, group_size)\n    return (x.astype(np.float32) @ w).astype(np.float64)"),
    ("matmul drops the last K row",
     "return x.astype(np.float64) @ w", "return x.astype(np.float64)[:, :-1] @ w[:-1]"),
    ("matmul rounds weights to fp16 first",
     "w = dequant(codes, scales, zeros, group_size).astype(np.float64)",
     "w = dequant(codes, scales, zeros, group_size).astype(np.float16).astype(np.float64)"),
]


def _edits(old, new):
    return old if new is None else [(old, new)]


def _load_mutant(old, new):
    src = open(SRC_PATH).read()
    for a, b in _edits(old, new):
        assert src.count(a) >= 1, f"mutation anchor not found: {a!r}"
        src = src.replace(a, b)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def test_mutation_anchors_present():
    src = open(SRC_PATH).read()
    for name, old, new in MUTANTS:
        for a, _ in _edits(old, new):
            assert src.count(a) >= 1, name


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    mod = _load_mutant(old, new)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except Exception:            # a wrong value or a crash both expose the mutant
            caught.append(pin.__name__)
    assert caught, f"no pin caught the mutant: {name}"
