"""Plain CPU oracle for the index-production step (top-k over indexer logits).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline may import or run this module.  The HIP library never calls it and
shares no code with it.

What is computed.  Each query row s has indexer logits over the kv rows and a
key range [ks[s], ke[s]) (its sequence's start and its causal end).  The
selection is the top-k of the logits inside the range, with k capped at the
range length n = ke - ks, padded back to the fixed width K with -1:

    n      = max(0, ke[s] - ks[s])
    m      = min(K, n)
    chosen = the m positions j in [ks, ke) with the largest logits[s, j],
             ties broken toward the smaller j
    out[s] = chosen in ascending j, then K - m entries of -1

Sources (page titles and sections):

  * Megatron-Bridge PR #17, "GLM-5 DSA option: tilelang (2/2)", Bug fixes:
    a top-k of fixed width over a packed sequence shorter than that width
    fails, so k is capped at the logits' row length and the selection is padded
    back to the fixed top-k width with the -1 sentinel, keeping the shape the
    attention kernel expects; the same section names the per-query starts and
    ends of the key range.

Readings where the pages leave the step open (each listed in the design
notes): the pages' top-k comes from a library call whose output order and tie
rule they do not state; the attention that consumes the indices treats its
slots as a set, so the order chosen here is ascending kv position and ties
go to the smaller position, which makes the result unique.  Logits are fp32
and must be finite (a NaN has no place in the order); the oracle raises on
one.  A range past the logits' row is clipped to it.
"""
from __future__ import annotations

import numpy as np


class TopkInputError(ValueError):
    """Raised on logits that are not finite or ranges that are malformed."""


def select_row(row: np.ndarray, ks: int, ke: int, K: int) -> np.ndarray:
    """One query row: the chosen kv positions, ascending, padded with -1 to K.

    A direct reading of the definition: sort the range by (logit descending,
    position ascending), keep the first min(K, n), list them ascending."""
    n_kv = row.shape[0]
    ks = max(0, int(ks))
    ke = min(n_kv, int(ke))
    out = np.full(K, -1, dtype=np.int32)
    if ke <= ks:
        return out
    seg = np.asarray(row[ks:ke], dtype=np.float64)
    if not np.all(np.isfinite(seg)):
        raise TopkInputError("logits must be finite")
    pos = np.arange(ks, ke, dtype=np.int64)
    # lexsort: last key is primary -> logit descending, then position ascending
    order = np.lexsort((pos, -seg))
    m = min(K, ke - ks)
    chosen = np.sort(pos[order[:m]])
    out[:m] = chosen.astype(np.int32)
    return out


def topk_indices(logits: np.ndarray, ks: np.ndarray, ke: np.ndarray, K: int) -> np.ndarray:
    """[S, K] int32 selections for logits [S, S_kv] and ranges ks, ke [S]."""
    logits = np.asarray(logits)
    if logits.ndim != 2:
        raise TopkInputError("logits must be [S, S_kv]")
    S = logits.shape[0]
    if np.shape(ks) != (S,) or np.shape(ke) != (S,) or K < 1:
        raise TopkInputError("ks, ke must be [S] and K >= 1")
    return np.stack([select_row(logits[s], ks[s], ke[s], K) for s in range(S)]) if S else \
        np.zeros((0, K), dtype=np.int32)


def causal_ranges(seqlens) -> tuple[np.ndarray, np.ndarray]:
    """ks, ke of packed sequences: token p of a sequence starting at c sees
    kv rows [c, c + p + 1)."""
    ks, ke, c = [], [], 0
    for L in seqlens:
        for p in range(int(L)):
            ks.append(c)
            ke.append(c + p + 1)
        c += int(L)
    return np.asarray(ks, dtype=np.int32), np.asarray(ke, dtype=np.int32)
