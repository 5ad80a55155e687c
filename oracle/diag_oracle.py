"""Plain CPU oracle for the nonfinite diagnostics (count NaN / Inf entries;
replace only those entries from a reference, or with zero).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline may import or run this module.  The HIP library never calls it and
shares no code with it.

Source (page title and section): slime issue #2201, "GLM-5.2 SparseMLA
TileLang backward returns NaN gradients from finite inputs", Workarounds
tested.  The fallback there runs the fast backward, keeps dq / dkv when they
are finite, and otherwise recomputes the call with a reference and takes the
reference's values only at the nonfinite entries; writing zeros at those
entries was the diagnostic confinement patch.

What is computed, on the raw bits of bf16 (uint16) or fp32 (uint32) data:

    nonfinite[i] = value of x[i] is NaN or +-Inf          (numpy.isfinite)
    count        = number of i with nonfinite[i]
    replaced[i]  = ref[i] if nonfinite[i] else x[i]       (ref absent: +0)

bf16 bits are widened to fp32 exactly (the 16 bits become the high half), so
the classification is numpy's on the widened value.
"""
from __future__ import annotations

import numpy as np

DTYPES = ("bf16", "f32")


def _values(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        b = np.asarray(bits, dtype=np.uint16)
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    if dtype == "f32":
        return np.asarray(bits, dtype=np.uint32).view(np.float32)
    raise ValueError(f"dtype must be one of {DTYPES}")


def nonfinite_mask(bits: np.ndarray, dtype: str) -> np.ndarray:
    """True where the element is NaN or an infinity."""
    return ~np.isfinite(_values(bits, dtype))


def count_nonfinite(bits: np.ndarray, dtype: str) -> int:
    """Number of NaN / Inf elements."""
    return int(np.count_nonzero(nonfinite_mask(bits, dtype)))


def replace_nonfinite(bits: np.ndarray, ref_bits: np.ndarray | None, dtype: str):
    """(new bits, number replaced): ref's bits (or +0) at the nonfinite
    elements, the input's bits everywhere else."""
    bits = np.asarray(bits)
    m = nonfinite_mask(bits, dtype)
    out = bits.copy()
    out[m] = 0 if ref_bits is None else np.asarray(ref_bits, dtype=bits.dtype)[m]
    return out, int(np.count_nonzero(m))
