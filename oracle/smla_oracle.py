"""Plain fp64 CPU oracle for DSA sparse-MLA attention, forward and backward.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline may import or run this module.  The HIP library never calls it and
shares no code with it; its job is to be slow, plain and checkable by eye.

What is computed (absorbed-latent layout, one KV group shared by all heads):

  For every query token s, J(s) is the list of its index slots that hold a
  row, in slot order; slots equal to -1 are padding and are skipped.  Each
  kept slot is its own softmax term, so a row listed twice counts twice.
  Keys are the whole 576-wide kv rows, values are their first 512 columns.

  forward, for every head h of token s:
      z_k  = scale * <q[s,h,:], kv[J_k, :]>             (all 576 columns)
      m    = max_k z_k                (m = 0 when J(s) is empty)
      l    = sum_k exp(z_k - m)       (l >= 1 whenever J(s) is not empty)
      lse  = m + ln(max(l, 1e-30))
      p_k  = exp(z_k - lse)
      out  = sum_k p_k * kv[J_k, :512]  (exactly 0 when J(s) is empty)

  backward, given dout and the forward's out/p:
      delta = <dout[s,h,:], out[s,h,:]>
      dp_k  = <dout[s,h,:], kv[J_k, :512]>
      ds_k  = p_k * (dp_k - delta)
      dq[s,h,:]          = scale * sum_k ds_k * kv[J_k, :]
      dkv[J_k, :]       += scale * ds_k * q[s,h,:]
      dkv[J_k, :512]    += p_k * dout[s,h,:]

Sources (page titles and sections):
  * slime issue #2201, "GLM-5.2 SparseMLA TileLang backward returns NaN
    gradients from finite inputs", sections Strongest repro evidence and
    Suspected area: the backward call takes (q, kv, out, dout, indices, lse,
    sm_scale) and returns (dq, dkv); the value width D=512 is fixed; dkv is
    accumulated through the indices; the check it calls for is a plain
    PyTorch-style reference over the same active positions.
  * miles PR #2079 digest, "fix GLM-5 sparse-MLA kernel -1 index OOB and NaN
    gradients", section 实现拆解 items 1-3 and the key code snippets: a slot is
    valid iff its index is not -1; padding slots contribute exactly zero to
    scores, probabilities, output and dkv; the key is the 512 latent columns
    plus the 64-wide tail; the value is the 512 latent columns; the softmax
    denominator (relative to the running max) is floored at 1e-30, which is a
    no-op on any row with a valid slot (its largest term is exp(0)=1) and
    makes an all-padding row output exactly zero with a finite LSE.
  * The gradient formulas (delta, P recompute, dP, dS, dQ, dKV) are the
    standard softmax-attention backward; they follow from the forward above
    by the chain rule, and the tests pin them by finite differences.

Parity pins for every function are in tests/test_oracle_*.py.  The one value
that no pin fixes is the LSE of an all-padding row: the pages only say it is
no longer -inf; this oracle takes the running max as 0 there, giving
lse = ln(1e-30) (parity unpinned for that single value).
"""
from __future__ import annotations

import math

import numpy as np

SUMEXP_FLOOR = 1e-30
EMPTY_ROW_LSE = math.log(SUMEXP_FLOOR)   # ln(1e-30) = -69.07755278982137


class OracleInputError(ValueError):
    """Raised when an index is neither -1 nor a row of kv."""


def _squeeze_group(kv: np.ndarray, idx: np.ndarray):
    """Accept kv [S_kv, DK] or [S_kv, 1, DK] and idx [S, K] or [S, 1, K]
    (one KV group); return the 2-D views."""
    if kv.ndim == 3:
        if kv.shape[1] != 1:
            raise OracleInputError("only one KV group is supported")
        kv = kv[:, 0, :]
    if idx.ndim == 3:
        if idx.shape[1] != 1:
            raise OracleInputError("only one KV group is supported")
        idx = idx[:, 0, :]
    return kv, idx


def valid_slots(idx_row: np.ndarray, s_kv: int) -> np.ndarray:
    """J(s): the rows listed by the non-padding slots of one index row, in slot
    order, duplicates kept.  A slot is padding iff it holds -1.  Any other value
    outside [0, s_kv) violates the input contract and raises."""
    row = np.asarray(idx_row).astype(np.int64)
    keep = row != -1
    J = row[keep]
    if J.size and (J.min() < 0 or J.max() >= s_kv):
        raise OracleInputError("index outside {-1} U [0, S_kv)")
    return J


def touched_rows(idx: np.ndarray, s_kv: int) -> np.ndarray:
    """Boolean mask over kv rows: True for every row some valid slot selects.
    These are exactly the rows whose dkv can be nonzero."""
    _, idx = _squeeze_group(np.zeros((s_kv, 1)), idx)
    flat = idx.reshape(-1).astype(np.int64)
    flat = flat[flat != -1]
    if flat.size and (flat.min() < 0 or flat.max() >= s_kv):
        raise OracleInputError("index outside {-1} U [0, S_kv)")
    mask = np.zeros(s_kv, dtype=bool)
    mask[flat] = True
    return mask


def token_forward(q_s: np.ndarray, rows: np.ndarray, scale: float, d_v: int):
    """Forward for one token.

    q_s  [H, DK] float64, rows [n, DK] float64 = kv[J(s)] (n may be 0).
    Returns out [H, d_v], lse [H], p [H, n].
    """
    H = q_s.shape[0]
    n = rows.shape[0]
    if n == 0:
        return (np.zeros((H, d_v)), np.full(H, EMPTY_ROW_LSE), np.zeros((H, 0)))
    z = scale * (q_s @ rows.T)                      # [H, n] scores over all DK columns
    m = z.max(axis=1)                               # running max of the row
    l = np.exp(z - m[:, None]).sum(axis=1)          # >= 1: the max term is exp(0)
    lse = m + np.log(np.maximum(l, SUMEXP_FLOOR))
    p = np.exp(z - lse[:, None])
    out = p @ rows[:, :d_v]                         # value = the first d_v columns
    return out, lse, p


def token_backward(q_s, rows, dout_s, out_s, p, scale, d_v):
    """Backward for one token, given its probabilities p [H, n] and out [H, d_v].

    Returns dq_s [H, DK] and the per-slot dkv contributions [n, DK].
    """
    H, DK = q_s.shape
    n = rows.shape[0]
    if n == 0:
        return np.zeros((H, DK)), np.zeros((0, DK))
    delta = (dout_s * out_s).sum(axis=1)             # [H]  rowsum(dO * O)
    dp = dout_s @ rows[:, :d_v].T                   # [H, n] dO . V^T
    ds = p * (dp - delta[:, None])                  # [H, n]
    dq_s = scale * (ds @ rows)                      # [H, DK]
    contrib = scale * (ds.T @ q_s)                  # [n, DK]  dS^T . Q  (key part)
    contrib[:, :d_v] += p.T @ dout_s                # [n, d_v] P^T . dO  (value part)
    return dq_s, contrib


def _as_f64(x):
    return np.asarray(x, dtype=np.float64)


def sparse_mla_fwd(q, kv, idx, sm_scale, d_v=512, tokens=None):
    """out [S, H, d_v], lse [S, H] (natural log) for every token, or only for
    the listed `tokens` (then the outputs have len(tokens) rows)."""
    q = _as_f64(q)
    kv, idx = _squeeze_group(_as_f64(kv), np.asarray(idx))
    S, H, DK = q.shape
    toks = range(S) if tokens is None else list(tokens)
    out = np.zeros((len(toks), H, d_v))
    lse = np.zeros((len(toks), H))
    for i, s in enumerate(toks):
        J = valid_slots(idx[s], kv.shape[0])
        o, l, _ = token_forward(q[s], kv[J], sm_scale, d_v)
        out[i], lse[i] = o, l
    return out, lse


def _scatter_add(dkv, J, contrib):
    if J.size == 0:
        return
    if np.unique(J).size == J.size:
        dkv[J] += contrib
    else:                                           # repeated rows: unbuffered add
        np.add.at(dkv, J, contrib)


def sparse_mla_bwd(q, kv, dout, idx, sm_scale, d_v=512, out=None, lse=None,
                   tokens=None, rows=None):
    """Gradients (dq [S, H, DK], dkv [S_kv, DK]) of the loss sum(dout * out).

    By default out and p are recomputed here in fp64 (the exact gradient of
    sparse_mla_fwd).  If `out` and `lse` are given (the forward's saved
    outputs, as the backward call on the pages receives them), delta uses the
    given out and p = exp(z - lse) uses the given lse instead.

    `tokens` limits dq to those tokens (dq then has len(tokens) rows) and
    `rows` limits dkv to those kv rows (dkv then has len(rows) rows); dkv of a
    row is always summed over every token that selects it.
    """
    q = _as_f64(q)
    dout = _as_f64(dout)
    kv, idx = _squeeze_group(_as_f64(kv), np.asarray(idx))
    S, H, DK = q.shape
    S_kv = kv.shape[0]
    supplied = out is not None
    if supplied:
        out = _as_f64(out)
        lse = _as_f64(lse)

    want_dq = np.ones(S, dtype=bool) if tokens is None else np.isin(np.arange(S), tokens)
    if rows is None:
        want_rows = np.ones(S_kv, dtype=bool)
    else:
        want_rows = np.zeros(S_kv, dtype=bool)
        want_rows[np.asarray(rows, dtype=np.int64)] = True
    dq = np.zeros((S, H, DK))
    dkv = np.zeros((S_kv, DK))
    for s in range(S):
        J = valid_slots(idx[s], S_kv)
        need_dkv = J.size > 0 and bool(want_rows[J].any())
        if not (want_dq[s] or need_dkv):
            continue
        R = kv[J]
        if supplied:
            z = sm_scale * (q[s] @ R.T)
            p = np.exp(z - lse[s][:, None])
            o = out[s]
        else:
            o, _, p = token_forward(q[s], R, sm_scale, d_v)
        dq_s, contrib = token_backward(q[s], R, dout[s], o, p, sm_scale, d_v)
        dq[s] = dq_s
        if need_dkv:
            _scatter_add(dkv, J, contrib)
    if tokens is not None:
        dq = dq[list(tokens)]
    if rows is not None:
        dkv = dkv[np.asarray(rows, dtype=np.int64)]
    return dq, dkv
