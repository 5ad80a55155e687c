"""Pins for the top-k index-production oracle (CPU only).

The oracle is held to things other than itself: torch.topk (an independent
library routine) on tie-free rows, a rank-count formulation of the same
selection on rows full of ties, the pages' cap-and-pad rule on short rows
(Megatron-Bridge PR #17, "GLM-5 DSA option: tilelang (2/2)", Bug fixes), and
invariances the definition implies.  A planted mistake (ties to the larger
position, or an off-by-one range) must fail a pin.
"""
import numpy as np
import pytest
import torch

from oracle import TopkInputError, causal_ranges, select_row, topk_indices


def _rank_select(row, ks, ke, K):
    """Position j is chosen iff fewer than m positions of the range beat it
    (a larger logit, or an equal logit at a smaller position)."""
    n = max(0, ke - ks)
    m = min(K, n)
    chosen = []
    for j in range(ks, ke):
        beat = sum(1 for i in range(ks, ke) if row[i] > row[j] or (row[i] == row[j] and i < j))
        if beat < m:
            chosen.append(j)
    return np.array(chosen + [-1] * (K - len(chosen)), dtype=np.int32)


def test_matches_torch_topk_on_tie_free_rows():
    rng = np.random.default_rng(0)
    S_kv, K = 300, 64
    logits = rng.standard_normal((40, S_kv)).astype(np.float32)
    ks = rng.integers(0, 100, 40).astype(np.int32)
    ke = (ks + rng.integers(0, 200, 40)).astype(np.int32)
    got = topk_indices(logits, ks, ke, K)
    for s in range(40):
        n = ke[s] - ks[s]
        m = min(K, n)
        if m == 0:
            assert (got[s] == -1).all()
            continue
        seg = torch.from_numpy(logits[s, ks[s]:ke[s]].astype(np.float64))
        ref = np.sort(torch.topk(seg, m).indices.numpy() + ks[s])
        np.testing.assert_array_equal(got[s, :m], ref)
        assert (got[s, m:] == -1).all()


def test_rank_formulation_on_rows_with_ties():
    rng = np.random.default_rng(1)
    for _ in range(60):
        S_kv = int(rng.integers(1, 40))
        K = int(rng.integers(1, 12))
        row = rng.integers(-2, 3, S_kv).astype(np.float32)   # heavy ties
        ks = int(rng.integers(0, S_kv))
        ke = int(rng.integers(ks, S_kv + 1))
        np.testing.assert_array_equal(select_row(row, ks, ke, K), _rank_select(row, ks, ke, K))


def test_short_rows_take_the_whole_range_then_pad():
    """The pages' fix: k is capped at the row length and the selection is
    padded back to the fixed width with -1."""
    rng = np.random.default_rng(2)
    ks, ke = causal_ranges([5, 3])
    logits = rng.standard_normal((8, 8)).astype(np.float32)
    got = topk_indices(logits, ks, ke, 6)
    for s in range(8):
        n = ke[s] - ks[s]
        np.testing.assert_array_equal(got[s, :n], np.arange(ks[s], ke[s]))
        assert (got[s, n:] == -1).all()
    assert got.shape == (8, 6) and got.dtype == np.int32


def test_causal_ranges_of_packed_sequences():
    ks, ke = causal_ranges([2, 3])
    np.testing.assert_array_equal(ks, [0, 0, 2, 2, 2])
    np.testing.assert_array_equal(ke, [1, 2, 3, 4, 5])


def test_invariances():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((16, 120)).astype(np.float32)
    ks = np.zeros(16, dtype=np.int32) + 10
    ke = np.arange(16, dtype=np.int32) * 7 + 20
    base = topk_indices(logits, ks, ke, 24)
    # values outside the range do not matter
    other = logits.copy()
    other[:, :10] = 1e6
    for s in range(16):
        other[s, ke[s]:] = 1e6
    np.testing.assert_array_equal(topk_indices(other, ks, ke, 24), base)
    # a strictly increasing map of the values keeps the selection
    np.testing.assert_array_equal(topk_indices(np.exp(logits / 4).astype(np.float64), ks, ke, 24),
                                  base)
    # a range past the row is clipped to it
    np.testing.assert_array_equal(topk_indices(logits, ks, ke + 1000, 24)[0],
                                  topk_indices(logits, ks, np.full(16, 120, np.int32), 24)[0])


def test_nonfinite_logits_are_rejected():
    row = np.array([0.0, np.nan, 1.0], dtype=np.float32)
    with pytest.raises(TopkInputError):
        select_row(row, 0, 3, 2)


def test_planted_mistakes_fail_a_pin():
    """Ties to the larger position, and a range that drops its last element,
    each disagree with the rank formulation on some row."""
    def ties_high(row, ks, ke, K):
        seg = row[ks:ke].astype(np.float64)
        pos = np.arange(ks, ke)
        order = np.lexsort((-pos, -seg))
        m = min(K, ke - ks)
        out = np.full(K, -1, np.int32)
        out[:m] = np.sort(pos[order[:m]])
        return out

    def short_range(row, ks, ke, K):
        return select_row(row, ks, max(ks, ke - 1), K)

    rng = np.random.default_rng(4)
    for bad in (ties_high, short_range):
        found = False
        for _ in range(50):
            row = rng.integers(-1, 2, 20).astype(np.float32)
            ks, ke, K = 2, 18, 5
            if not np.array_equal(bad(row, ks, ke, K), _rank_select(row, ks, ke, K)):
                found = True
                break
        assert found, bad.__name__
