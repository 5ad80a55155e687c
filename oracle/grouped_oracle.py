"""fp64 CPU oracle for sparse-MLA attention with several KV groups.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline may import or run this module; it shares no code with the HIP
library.

The kernel excerpts of the miles PR #2079 digest ("fix GLM-5 sparse-MLA kernel
-1 index OOB and NaN gradients", key code snippets) address the index tensor
and the kv tensor with a kv-group coordinate that comes from the query head
block (the forward's g_i, the backward's head block over heads per group).
Reading: the H query heads split into G equal contiguous blocks of H / G, and
block g attends over kv group g with its own index rows.  With
    q [S, H, 576], kv [S_kv, G, 576], idx [S, G, K], dout [S, H, 512],
head h of token s is single-group attention over kv[:, g] with index row
idx[s, g], g = h // (H / G); dkv[:, g] collects the gradients of the heads of
block g only.  Each group is one call of the single-group oracle.
"""
from __future__ import annotations

import numpy as np

from .smla_oracle import OracleInputError, sparse_mla_bwd, sparse_mla_fwd


def _groups(q: np.ndarray, kv: np.ndarray, idx: np.ndarray):
    if kv.ndim != 3 or idx.ndim != 3 or kv.shape[1] != idx.shape[1]:
        raise OracleInputError("grouped inputs: kv [S_kv, G, DK] and idx [S, G, K]")
    G = kv.shape[1]
    H = q.shape[1]
    if H % G:
        raise OracleInputError("heads must split evenly over the kv groups")
    return G, H // G


def sparse_mla_fwd_grouped(q, kv, idx, sm_scale, d_v=512):
    """out [S, H, d_v], lse [S, H] for grouped inputs."""
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    idx = np.asarray(idx)
    G, hg = _groups(q, kv, idx)
    S, H, _ = q.shape
    out = np.zeros((S, H, d_v))
    lse = np.zeros((S, H))
    for g in range(G):
        heads = slice(g * hg, (g + 1) * hg)
        out[:, heads], lse[:, heads] = sparse_mla_fwd(q[:, heads], kv[:, g], idx[:, g], sm_scale,
                                                      d_v=d_v)
    return out, lse


def sparse_mla_bwd_grouped(q, kv, dout, idx, sm_scale, d_v=512, out=None, lse=None):
    """dq [S, H, DK], dkv [S_kv, G, DK] of the loss sum(dout * out); `out` and
    `lse` as in sparse_mla_bwd (the forward's saved outputs, optional)."""
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    idx = np.asarray(idx)
    G, hg = _groups(q, kv, idx)
    dq = np.zeros(q.shape)
    dkv = np.zeros(kv.shape)
    for g in range(G):
        heads = slice(g * hg, (g + 1) * hg)
        kw = {}
        if out is not None:
            kw = {"out": np.asarray(out, dtype=np.float64)[:, heads],
                  "lse": np.asarray(lse, dtype=np.float64)[:, heads]}
        dq[:, heads], dkv[:, g] = sparse_mla_bwd(q[:, heads], kv[:, g], dout[:, heads], idx[:, g],
                                                 sm_scale, d_v=d_v, **kw)
    return dq, dkv
