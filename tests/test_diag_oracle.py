"""Pins for the nonfinite-diagnostics oracle (CPU).

The classification is fixed by IEEE-754: an element is NaN or an infinity
exactly when all its exponent bits are ones (binary32: bits 23..30; bfloat16,
the high half of a binary32: bits 7..14).  The tables below are written out
by hand from that rule, not computed by the oracle."""
import numpy as np
import pytest

from oracle import count_nonfinite, nonfinite_mask, replace_nonfinite
from workloads import synth

# (bits, is_nonfinite, what)
BF16_TABLE = [
    (0x0000, False, "+0"), (0x8000, False, "-0"), (0x0001, False, "smallest subnormal"),
    (0x007F, False, "largest subnormal"), (0x0080, False, "smallest normal"),
    (0x3F80, False, "1.0"), (0xBF80, False, "-1.0"), (0x7F7F, False, "largest finite"),
    (0xFF7F, False, "most negative finite"), (0x7F00, False, "2^127"),
    (0x7F80, True, "+inf"), (0xFF80, True, "-inf"), (0x7FC0, True, "quiet NaN"),
    (0xFFC0, True, "negative quiet NaN"), (0x7F81, True, "signalling NaN"),
    (0xFFFF, True, "all ones"), (0x7FFF, True, "NaN, max payload"),
]
F32_TABLE = [
    (0x00000000, False, "+0"), (0x80000000, False, "-0"), (0x00000001, False, "smallest subnormal"),
    (0x007FFFFF, False, "largest subnormal"), (0x3F800000, False, "1.0"),
    (0x7F7FFFFF, False, "largest finite"), (0xFF7FFFFF, False, "most negative finite"),
    (0x7F000000, False, "2^127"), (0x7F800000, True, "+inf"), (0xFF800000, True, "-inf"),
    (0x7FC00000, True, "quiet NaN"), (0x7F800001, True, "signalling NaN"),
    (0xFFFFFFFF, True, "all ones"), (0x7FFFFFFF, True, "NaN, max payload"),
]


@pytest.mark.parametrize("dtype,table,np_t", [("bf16", BF16_TABLE, np.uint16),
                                               ("f32", F32_TABLE, np.uint32)])
def test_classification_table(dtype, table, np_t):
    bits = np.array([b for b, _, _ in table], dtype=np_t)
    want = np.array([f for _, f, _ in table])
    got = nonfinite_mask(bits, dtype)
    for (b, f, what), g in zip(table, got):
        assert g == f, f"{dtype} {what} ({b:#x})"
    assert count_nonfinite(bits, dtype) == int(want.sum())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_replace_takes_the_reference_only_at_nonfinite_entries(dtype):
    bits, ref = synth.planted_nonfinite(10007, dtype, frac=0.05, seed=3)
    width = 16 if dtype == "bf16" else 32
    exp_mask = (0x7F80 if width == 16 else 0x7F800000)
    planted = (bits.astype(np.uint64) & exp_mask) == exp_mask     # the exponent rule, restated
    new, n = replace_nonfinite(bits, ref, dtype)
    assert n == int(planted.sum()) == count_nonfinite(bits, dtype) > 0
    assert np.array_equal(new[planted], ref[planted])
    assert np.array_equal(new[~planted], bits[~planted])
    assert count_nonfinite(new, dtype) == 0
    zero, n0 = replace_nonfinite(bits, None, dtype)
    assert n0 == n and np.all(zero[planted] == 0) and np.array_equal(zero[~planted], bits[~planted])


def test_replace_with_itself_and_on_finite_data():
    bits, _ = synth.planted_nonfinite(999, "bf16", frac=0.1, seed=4)
    same, n = replace_nonfinite(bits, bits, "bf16")
    assert np.array_equal(same, bits) and n == count_nonfinite(bits, "bf16")
    clean, _ = synth.planted_nonfinite(999, "f32", frac=0.0, seed=5)
    out, n = replace_nonfinite(clean, clean[::-1].copy(), "f32")
    assert n == 0 and np.array_equal(out, clean)


def test_counts_add_over_concatenation():
    a, _ = synth.planted_nonfinite(1000, "f32", frac=0.03, seed=6)
    b, _ = synth.planted_nonfinite(777, "f32", frac=0.2, seed=7)
    assert count_nonfinite(np.concatenate([a, b]), "f32") == count_nonfinite(a, "f32") + count_nonfinite(b, "f32")
    assert count_nonfinite(a, "f32") == 30 and count_nonfinite(b, "f32") == 155   # round(frac * n)


def test_planted_mistakes_are_caught():
    """Plausible wrong classifiers each disagree with the hand-written table."""
    bits16 = np.array([b for b, _, _ in BF16_TABLE], dtype=np.uint16)
    want16 = np.array([f for _, f, _ in BF16_TABLE])
    wrong = {
        "isnan only": lambda b: np.isnan((b.astype(np.uint32) << 16).view(np.float32)),
        "isinf only": lambda b: np.isinf((b.astype(np.uint32) << 16).view(np.float32)),
        "widened by 8 bits": lambda b: ~np.isfinite((b.astype(np.uint32) << 8).view(np.float32)),
        "sign bit in the mask": lambda b: (b & 0xFF80) == 0xFF80,
        "magnitude test": lambda b: np.abs((b.astype(np.uint32) << 16).view(np.float32)) > 3.0e38,
    }
    for name, f in wrong.items():
        assert not np.array_equal(f(bits16), want16), name
