"""Pins for the fp64 oracle: each test checks it against something other than
itself -- a library routine (dense causal attention, torch autograd), central
finite differences, closed forms, invariants or brute force over index sets.

The mutation tests in test_oracle_mutations.py plant mistakes into a copy of
the oracle and check that these pins catch them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (EMPTY_ROW_LSE, SUMEXP_FLOOR, OracleInputError,
                    sparse_mla_bwd, sparse_mla_fwd, touched_rows)
from workloads import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")


def rand_inputs(rng, S, H, S_kv, DK, DV, scale_q=1.0):
    q = rng.standard_normal((S, H, DK)) * scale_q
    kv = rng.standard_normal((S_kv, DK))
    dout = rng.standard_normal((S, H, DV))
    return q, kv, dout


def causal_full_idx(rng, seqlens, K):
    S = sum(seqlens)
    idx = np.full((S, K), -1, dtype=np.int64)
    start = 0
    for n in seqlens:
        for p in range(n):
            idx[start + p, : p + 1] = rng.permutation(p + 1) + start
        start += n
    return idx


# ---------------------------------------------------------------------------
# 1. Reduction to a textbook routine: dense causal attention per sequence.
# ---------------------------------------------------------------------------

def dense_causal_torch(q, kv, dout, seqlens, scale, DV):
    """Per-sequence dense causal softmax attention in torch fp64, with kv as a
    leaf used both as keys (all columns) and values (first DV columns).
    Returns out, lse, dq, dkv from torch's own softmax/logsumexp/autograd."""
    qt = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    kvt = torch.tensor(kv, dtype=torch.float64, requires_grad=True)
    outs, lses = [], []
    start = 0
    for n in seqlens:
        qs = qt[start:start + n].transpose(0, 1)            # [H, n, DK]
        ks = kvt[start:start + n]                           # [n, DK]
        sc = scale * torch.matmul(qs, ks.t())               # [H, n, n]
        causal = torch.ones(n, n, dtype=torch.bool).tril()
        sc = sc.masked_fill(~causal, float("-inf"))
        lses.append(torch.logsumexp(sc, dim=-1).transpose(0, 1))
        pr = torch.softmax(sc, dim=-1)
        outs.append(torch.matmul(pr, ks[:, :DV]).transpose(0, 1))
        start += n
    out = torch.cat(outs, 0)
    lse = torch.cat(lses, 0)
    (out * torch.tensor(dout)).sum().backward()
    return (out.detach().numpy(), lse.detach().numpy(), qt.grad.numpy(), kvt.grad.numpy())


@pytest.mark.parametrize("DK,DV", [(576, 512), (12, 8)])
def test_dense_causal_reduction(DK, DV):
    rng = np.random.default_rng(11)
    seqlens, H, K = [5, 9, 3, 1], 3, 12
    S = sum(seqlens)
    q, kv, dout = rand_inputs(rng, S, H, S, DK, DV)
    idx = causal_full_idx(rng, seqlens, K)
    scale = 1 / math.sqrt(192)
    out, lse = sparse_mla_fwd(q, kv, idx, scale, d_v=DV)
    dq, dkv = sparse_mla_bwd(q, kv, dout, idx, scale, d_v=DV)
    r_out, r_lse, r_dq, r_dkv = dense_causal_torch(q, kv, dout, seqlens, scale, DV)
    np.testing.assert_allclose(out, r_out, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, r_lse, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dq, r_dq, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dkv, r_dkv, rtol=1e-11, atol=1e-12)


def test_dense_causal_matches_sdpa():
    """Same reduction against torch's scaled_dot_product_attention (fp64)."""
    rng = np.random.default_rng(12)
    seqlens, H, K, DK, DV = [7, 4], 2, 8, 16, 16
    S = sum(seqlens)
    q, kv, _ = rand_inputs(rng, S, H, S, DK, DV)
    idx = causal_full_idx(rng, seqlens, K)
    scale = 0.37
    out, _ = sparse_mla_fwd(q, kv, idx, scale, d_v=DV)
    start = 0
    for n in seqlens:
        qs = torch.tensor(q[start:start + n]).transpose(0, 1)[None]
        ks = torch.tensor(kv[start:start + n])[None, None].expand(1, H, n, DK)
        vs = ks[..., :DV]
        ref = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, is_causal=True,
                                                               scale=scale)
        np.testing.assert_allclose(out[start:start + n], ref[0].transpose(0, 1).numpy(),
                                   rtol=1e-12, atol=1e-12)
        start += n


def test_dense_causal_on_generated_workload():
    """The tiny generated workload's first 64 rows list every causal position
    (row s has s+1 <= 64 candidates), so they equal dense causal attention."""
    w = synth.tiny()
    q = synth.bf16_bits_to_f64(w.q)[:64]
    kv = synth.bf16_bits_to_f64(w.kv)[:64]
    dout = synth.bf16_bits_to_f64(w.dout)[:64]
    idx = w.idx[:64]
    out, lse = sparse_mla_fwd(q, kv, idx, w.sm_scale)
    r_out, r_lse, _, _ = dense_causal_torch(q, kv, dout, [64], w.sm_scale, 512)
    np.testing.assert_allclose(out, r_out, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, r_lse, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# 2. Brute force against torch autograd over an explicit gather formulation.
# ---------------------------------------------------------------------------

def gather_autograd_torch(q, kv, dout, idx, scale, DV):
    """Explicit gather + masked_fill(-inf) + softmax in torch fp64 with kv as
    a leaf; rows with no valid slot are excluded from torch's softmax (it
    would produce NaN) and their out is 0.  Returns out, lse (NaN where empty),
    dq, dkv."""
    qt = torch.tensor(q, requires_grad=True)
    kvt = torch.tensor(kv, requires_grad=True)
    it = torch.tensor(idx, dtype=torch.long)
    valid = it != -1
    gathered = kvt[it.clamp(min=0)]                          # [S, K, DK]
    sc = scale * torch.einsum("shd,skd->shk", qt, gathered)
    sc = sc.masked_fill(~valid[:, None, :], float("-inf"))
    nonempty = valid.any(dim=1)
    S, H = q.shape[:2]
    out = torch.zeros(S, H, DV, dtype=torch.float64)
    lse = torch.full((S, H), float("nan"), dtype=torch.float64)
    pr = torch.softmax(sc[nonempty], dim=-1)
    out_ne = torch.einsum("shk,skd->shd", pr, gathered[nonempty][..., :DV])
    out = out.index_put((nonempty.nonzero()[:, 0],), out_ne)
    lse = lse.index_put((nonempty.nonzero()[:, 0],), torch.logsumexp(sc[nonempty], dim=-1))
    (out * torch.tensor(dout)).sum().backward()
    return out.detach().numpy(), lse.detach().numpy(), qt.grad.numpy(), kvt.grad.numpy()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_autograd_with_padding_and_duplicates(seed):
    rng = np.random.default_rng(100 + seed)
    S, H, S_kv, K, DK, DV = 9, 2, 7, 6, 10, 6
    q, kv, dout = rand_inputs(rng, S, H, S_kv, DK, DV, scale_q=2.0)
    idx = rng.integers(0, S_kv, size=(S, K))                 # duplicates likely
    idx[rng.random((S, K)) < 0.35] = -1                      # -1 anywhere in a row
    idx[3] = -1                                              # an all-padding row
    scale = 0.8
    out, lse = sparse_mla_fwd(q, kv, idx, scale, d_v=DV)
    dq, dkv = sparse_mla_bwd(q, kv, dout, idx, scale, d_v=DV)
    r_out, r_lse, r_dq, r_dkv = gather_autograd_torch(q, kv, dout, idx, scale, DV)
    np.testing.assert_allclose(out, r_out, rtol=1e-12, atol=1e-13)
    ne = ~np.isnan(r_lse)
    np.testing.assert_allclose(lse[ne], r_lse[ne], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dq, r_dq, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dkv, r_dkv, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# 3. Central finite differences of L = sum(dout * out).
# ---------------------------------------------------------------------------

def test_central_finite_differences():
    rng = np.random.default_rng(5)
    S, H, S_kv, K, DK, DV = 6, 2, 6, 4, 12, 8
    q, kv, dout = rand_inputs(rng, S, H, S_kv, DK, DV)
    idx = np.array([[0, -1, 2, 5], [-1, -1, -1, -1], [1, 1, -1, 3],
                    [4, 0, 2, -1], [5, -1, -1, -1], [3, 2, 1, 0]])
    scale = 0.6

    def loss(qq, kk):
        o, _ = sparse_mla_fwd(qq, kk, idx, scale, d_v=DV)
        return float((o * dout).sum())

    dq, dkv = sparse_mla_bwd(q, kv, dout, idx, scale, d_v=DV)
    h = 1e-6
    num_dq = np.zeros_like(q)
    for i in np.ndindex(q.shape):
        a, b = q.copy(), q.copy()
        a[i] += h
        b[i] -= h
        num_dq[i] = (loss(a, kv) - loss(b, kv)) / (2 * h)
    num_dkv = np.zeros_like(kv)
    for i in np.ndindex(kv.shape):
        a, b = kv.copy(), kv.copy()
        a[i] += h
        b[i] -= h
        num_dkv[i] = (loss(q, a) - loss(q, b)) / (2 * h)
    assert np.abs(num_dq - dq).max() <= 1e-7 * max(1.0, np.abs(dq).max())
    assert np.abs(num_dkv - dkv).max() <= 1e-7 * max(1.0, np.abs(dkv).max())
    assert np.all(dq[1] == 0.0)                 # the empty row has no gradient


def test_finite_differences_of_lse():
    """lse is the log-partition: d lse / d q[s,h] = scale * sum_k p_k kv[J_k],
    i.e. the probability-weighted key; checked by central differences."""
    rng = np.random.default_rng(6)
    S, H, S_kv, K, DK, DV = 3, 2, 5, 4, 9, 6
    q, kv, _ = rand_inputs(rng, S, H, S_kv, DK, DV)
    idx = np.array([[0, 4, -1, 2], [1, -1, 3, 3], [2, 2, 2, -1]])
    scale = 0.9
    _, lse = sparse_mla_fwd(q, kv, idx, scale, d_v=DV)
    h = 1e-6
    for s in range(S):
        J = idx[s][idx[s] != -1]
        for hh in range(H):
            z = scale * kv[J] @ q[s, hh]
            p = np.exp(z - lse[s, hh])
            expect = scale * (p @ kv[J])
            num = np.zeros(DK)
            for d in range(DK):
                a, b = q.copy(), q.copy()
                a[s, hh, d] += h
                b[s, hh, d] -= h
                num[d] = (sparse_mla_fwd(a, kv, idx, scale, d_v=DV)[1][s, hh]
                          - sparse_mla_fwd(b, kv, idx, scale, d_v=DV)[1][s, hh]) / (2 * h)
            np.testing.assert_allclose(num, expect, rtol=1e-6, atol=1e-8)


# ---------------------------------------------------------------------------
# 4. Closed forms.
# ---------------------------------------------------------------------------

def test_single_valid_slot():
    rng = np.random.default_rng(7)
    H, S_kv, DK, DV = 4, 5, 20, 16
    q, kv, dout = rand_inputs(rng, 1, H, S_kv, DK, DV)
    j = 3
    idx = np.array([[-1, j, -1, -1, -1]])
    scale = 0.5
    out, lse = sparse_mla_fwd(q, kv, idx, scale, d_v=DV)
    assert np.array_equal(out[0], np.broadcast_to(kv[j, :DV], (H, DV)))
    np.testing.assert_allclose(lse[0], scale * q[0] @ kv[j], rtol=1e-15, atol=1e-15)
    dq, dkv = sparse_mla_bwd(q, kv, dout, idx, scale, d_v=DV)
    assert np.abs(dq).max() < 1e-13
    expect = np.zeros(DK)
    expect[:DV] = dout[0].sum(axis=0)
    np.testing.assert_allclose(dkv[j], expect, rtol=1e-13, atol=1e-13)
    assert np.all(np.delete(dkv, j, axis=0) == 0.0)


def test_two_slots_sigmoid():
    rng = np.random.default_rng(8)
    H, DK, DV = 3, 10, 6
    q, kv, _ = rand_inputs(rng, 1, H, 2, DK, DV)
    scale = 1.3
    out, lse = sparse_mla_fwd(q, kv, np.array([[1, -1, 0]]), scale, d_v=DV)
    z0 = scale * q[0] @ kv[0]
    z1 = scale * q[0] @ kv[1]
    p0 = 1.0 / (1.0 + np.exp(z1 - z0))
    np.testing.assert_allclose(out[0], p0[:, None] * kv[0, :DV] + (1 - p0)[:, None] * kv[1, :DV],
                               rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse[0], np.logaddexp(z0, z1), rtol=1e-14, atol=1e-14)


def test_identical_keys_duplicates():
    """n copies of one row: p = 1/n each, out = v, lse = z + ln n, dq = 0,
    dkv[j] = sum_h [dout, 0]."""
    rng = np.random.default_rng(9)
    H, DK, DV, n = 2, 8, 5, 5
    q, kv, dout = rand_inputs(rng, 1, H, 3, DK, DV)
    j = 2
    idx = np.array([[j] * n + [-1, -1]])
    scale = 0.7
    out, lse = sparse_mla_fwd(q, kv, idx, scale, d_v=DV)
    np.testing.assert_allclose(out[0], np.broadcast_to(kv[j, :DV], (H, DV)), rtol=1e-14)
    np.testing.assert_allclose(lse[0], scale * q[0] @ kv[j] + math.log(n), rtol=1e-14)
    dq, dkv = sparse_mla_bwd(q, kv, dout, idx, scale, d_v=DV)
    assert np.abs(dq).max() < 1e-13
    expect = np.zeros(DK)
    expect[:DV] = dout[0].sum(axis=0)
    np.testing.assert_allclose(dkv[j], expect, rtol=1e-13, atol=1e-13)


def test_dkv_column_sums_closed_form():
    """sum_k ds_k = 0 for every (s,h) with a valid slot, hence
    sum_j dkv[j,:DV] = sum of dout over nonempty tokens and sum_j dkv[j,DV:] = 0."""
    w = synth.custom(S=40, H=4, K=24, S_kv=30, seed=3, dup_frac=0.1)
    q = synth.bf16_bits_to_f64(w.q)
    kv = synth.bf16_bits_to_f64(w.kv)
    dout = synth.bf16_bits_to_f64(w.dout)
    dq, dkv = sparse_mla_bwd(q, kv, dout, w.idx, w.sm_scale)
    nonempty = (w.idx != -1).any(axis=1)
    lhs = dkv.sum(axis=0)
    np.testing.assert_allclose(lhs[:512], dout[nonempty].sum(axis=(0, 1)), rtol=1e-11, atol=1e-10)
    assert np.abs(lhs[512:]).max() <= 1e-12 * np.abs(dkv[:, 512:]).sum()


# ---------------------------------------------------------------------------
# 5. Invariants.
# ---------------------------------------------------------------------------

def _small_case(seed=21):
    rng = np.random.default_rng(seed)
    S, H, S_kv, K, DK, DV = 7, 3, 9, 5, 14, 10
    q, kv, dout = rand_inputs(rng, S, H, S_kv, DK, DV)
    idx = np.stack([rng.choice(S_kv, K, replace=False) for _ in range(S)])
    idx[2, 1] = -1
    idx[5] = -1
    return q, kv, dout, idx, 0.45, DV


def test_permutation_invariance():
    q, kv, dout, idx, scale, DV = _small_case()
    rng = np.random.default_rng(1)
    perm = np.stack([rng.permutation(idx.shape[1]) for _ in range(idx.shape[0])])
    idx2 = np.take_along_axis(idx, perm, axis=1)
    for a, b in zip(sparse_mla_fwd(q, kv, idx, scale, d_v=DV),
                    sparse_mla_fwd(q, kv, idx2, scale, d_v=DV)):
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)
    for a, b in zip(sparse_mla_bwd(q, kv, dout, idx, scale, d_v=DV),
                    sparse_mla_bwd(q, kv, dout, idx2, scale, d_v=DV)):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_inserting_padding_changes_nothing():
    q, kv, dout, idx, scale, DV = _small_case()
    S, K = idx.shape
    wide = np.full((S, 3 * K), -1)
    rng = np.random.default_rng(2)
    for s in range(S):
        pos = np.sort(rng.choice(3 * K, K, replace=False))
        wide[s, pos] = idx[s]
    for a, b in zip(sparse_mla_fwd(q, kv, idx, scale, d_v=DV),
                    sparse_mla_fwd(q, kv, wide, scale, d_v=DV)):
        assert np.array_equal(a, b)
    for a, b in zip(sparse_mla_bwd(q, kv, dout, idx, scale, d_v=DV),
                    sparse_mla_bwd(q, kv, dout, wide, scale, d_v=DV)):
        assert np.array_equal(a, b)


def test_all_padding_rows_exact():
    q, kv, dout, idx, scale, DV = _small_case()
    out, lse = sparse_mla_fwd(q, kv, idx, scale, d_v=DV)
    dq, dkv = sparse_mla_bwd(q, kv, dout, idx, scale, d_v=DV)
    assert np.all(out[5] == 0.0) and np.all(dq[5] == 0.0)
    assert np.all(lse[5] == EMPTY_ROW_LSE) and np.isfinite(lse).all()
    # the empty row contributes nothing to dkv: changing its q/dout changes nothing
    q2, d2 = q.copy(), dout.copy()
    q2[5] += 100.0
    d2[5] -= 50.0
    _, dkv2 = sparse_mla_bwd(q2, kv, d2, idx, scale, d_v=DV)
    assert np.array_equal(dkv, dkv2)


def test_linearity_in_dout():
    q, kv, dout, idx, scale, DV = _small_case()
    rng = np.random.default_rng(3)
    d2 = rng.standard_normal(dout.shape)
    a, b = 1.7, -0.4
    g1 = sparse_mla_bwd(q, kv, dout, idx, scale, d_v=DV)
    g2 = sparse_mla_bwd(q, kv, d2, idx, scale, d_v=DV)
    g3 = sparse_mla_bwd(q, kv, a * dout + b * d2, idx, scale, d_v=DV)
    for x1, x2, x3 in zip(g1, g2, g3):
        np.testing.assert_allclose(x3, a * x1 + b * x2, rtol=1e-11, atol=1e-12)


def test_unselected_rows_exactly_zero_and_touched_set():
    q, kv, dout, idx, scale, DV = _small_case()
    _, dkv = sparse_mla_bwd(q, kv, dout, idx, scale, d_v=DV)
    brute = np.zeros(kv.shape[0], dtype=bool)
    for s in range(idx.shape[0]):
        for k in range(idx.shape[1]):
            if idx[s, k] != -1:
                brute[idx[s, k]] = True
    assert np.array_equal(touched_rows(idx, kv.shape[0]), brute)
    assert np.all(dkv[~brute] == 0.0)
    assert np.all(np.abs(dkv[brute]).sum(axis=1) > 0)


def test_supplied_out_lse_mode_equals_recompute():
    q, kv, dout, idx, scale, DV = _small_case()
    out, lse = sparse_mla_fwd(q, kv, idx, scale, d_v=DV)
    a = sparse_mla_bwd(q, kv, dout, idx, scale, d_v=DV)
    b = sparse_mla_bwd(q, kv, dout, idx, scale, d_v=DV, out=out, lse=lse)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-13)


# The supplied-out / lse branch away from its fixed point.  The backward call
# on the pages takes the forward's saved out and lse (slime issue #2201,
# Strongest repro evidence); with them given, p = exp(z - lse) reads the given
# lse and delta = <dout, out> the given out, so:
#   * lse + c multiplies p, dS, dq and every dkv contribution by exp(-c)
#     (delta does not move);
#   * out + E changes delta by <dout, E> only: dq[s,h] moves by
#     -scale <dout[s,h], E[s,h]> sum_k p_k kv[J_k] and each dkv[J_k] by
#     -scale p_k <dout[s,h], E[s,h]> q[s,h], with p the softmax of the
#     token's scores (torch's softmax here, not the oracle's).

def supplied_lse_shift_ok(mod, seed=23) -> bool:
    q, kv, dout, idx, scale, DV = _small_case(seed)
    out, lse = mod.sparse_mla_fwd(q, kv, idx, scale, d_v=DV)
    rng = np.random.default_rng(seed + 1)
    out = out + 0.3 * rng.standard_normal(out.shape)     # off the fixed point
    base = mod.sparse_mla_bwd(q, kv, dout, idx, scale, d_v=DV, out=out, lse=lse)
    c = 0.7                                              # one shift: dkv scales too
    shifted = mod.sparse_mla_bwd(q, kv, dout, idx, scale, d_v=DV, out=out, lse=lse + c)
    ok = all(np.allclose(y, math.exp(-c) * x, rtol=1e-12, atol=1e-14)
             for x, y in zip(base, shifted))
    cr = rng.uniform(-2.0, 2.0, size=lse.shape)          # per (token, head): dq row-wise
    dq_r, _ = mod.sparse_mla_bwd(q, kv, dout, idx, scale, d_v=DV, out=out, lse=lse + cr)
    ok = ok and np.allclose(dq_r, np.exp(-cr)[:, :, None] * base[0], rtol=1e-12, atol=1e-14)
    return bool(ok) and float(np.abs(base[0]).max()) > 0.0


def supplied_out_perturbation_ok(mod, seed=24) -> bool:
    q, kv, dout, idx, scale, DV = _small_case(seed)
    out, lse = mod.sparse_mla_fwd(q, kv, idx, scale, d_v=DV)
    rng = np.random.default_rng(seed + 1)
    E = rng.standard_normal(out.shape)
    dq0, dkv0 = mod.sparse_mla_bwd(q, kv, dout, idx, scale, d_v=DV, out=out, lse=lse)
    dq1, dkv1 = mod.sparse_mla_bwd(q, kv, dout, idx, scale, d_v=DV, out=out + E, lse=lse)
    S, H, DK = q.shape
    exp_dq = np.zeros_like(dq0)
    exp_dkv = torch.zeros((kv.shape[0], DK), dtype=torch.float64)
    for s in range(S):
        J = idx[s][idx[s] != -1]
        if J.size == 0:
            continue
        rows = torch.tensor(kv[J])
        qs = torch.tensor(q[s])
        p = torch.softmax(scale * qs @ rows.T, dim=-1)               # [H, n]
        d = torch.tensor((dout[s] * E[s]).sum(axis=1))               # <dout, E> per head
        exp_dq[s] = (-scale * d[:, None] * (p @ rows)).numpy()
        exp_dkv.index_add_(0, torch.tensor(J), -scale * (p * d[:, None]).T @ qs)
    return bool(np.allclose(dq1 - dq0, exp_dq, rtol=1e-9, atol=1e-12)
                and np.allclose(dkv1 - dkv0, exp_dkv.numpy(), rtol=1e-9, atol=1e-12)
                and float(np.abs(exp_dq).max()) > 0.0)


def test_supplied_lse_shift_scales_gradients():
    import oracle.smla_oracle as mod
    assert supplied_lse_shift_ok(mod)


def test_supplied_out_changes_delta_only():
    import oracle.smla_oracle as mod
    assert supplied_out_perturbation_ok(mod)


def test_sampled_tokens_and_rows_match_full():
    q, kv, dout, idx, scale, DV = _small_case()
    out, lse = sparse_mla_fwd(q, kv, idx, scale, d_v=DV)
    dq, dkv = sparse_mla_bwd(q, kv, dout, idx, scale, d_v=DV)
    toks = [6, 0, 5]
    rows = [8, 1, 4]
    o2, l2 = sparse_mla_fwd(q, kv, idx, scale, d_v=DV, tokens=toks)
    dq2, dkv2 = sparse_mla_bwd(q, kv, dout, idx, scale, d_v=DV, tokens=toks, rows=rows)
    assert np.array_equal(o2, out[toks]) and np.array_equal(l2, lse[toks])
    assert np.array_equal(dq2, dq[toks])
    np.testing.assert_allclose(dkv2, dkv[rows], rtol=1e-14, atol=1e-15)


def test_out_of_range_index_raises():
    q, kv, dout, idx, scale, DV = _small_case()
    bad = idx.copy()
    bad[0, 0] = kv.shape[0]
    with pytest.raises(OracleInputError):
        sparse_mla_fwd(q, kv, bad, scale, d_v=DV)
    bad[0, 0] = -2
    with pytest.raises(OracleInputError):
        sparse_mla_bwd(q, kv, dout, bad, scale, d_v=DV)


def test_group_dimension_accepted():
    q, kv, dout, idx, scale, DV = _small_case()
    a = sparse_mla_fwd(q, kv, idx, scale, d_v=DV)
    b = sparse_mla_fwd(q, kv[:, None, :], idx[:, None, :], scale, d_v=DV)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ---------------------------------------------------------------------------
# 6. Facts printed on the pages.
# ---------------------------------------------------------------------------

def test_pages_facts():
    facts = json.load(open(GOLDEN))
    assert SUMEXP_FLOOR == facts["sumexp_floor"]["value"]
    assert EMPTY_ROW_LSE == math.log(facts["sumexp_floor"]["value"])
    assert synth.D_LATENT == facts["value_width_D"]["value"]
    assert synth.D_ROPE == facts["rope_tail_width"]["value"]
    nan = facts["nan_counts_of_bad_call"]
    assert nan["dq"] % nan["row_width"] == 0 and nan["dkv"] % nan["row_width"] == 0
    # the production shape of the packed workload is the pages' H=8, topk=2048
    assert facts["production_shape"]["heads"] == 8 and facts["production_shape"]["topk"] == 2048


def test_floor_is_noop_on_real_rows():
    """Real rows have l >= 1 (their max term is exp(0)), so the 1e-30 floor
    never changes them: lse equals torch.logsumexp exactly up to rounding even
    for very negative logits."""
    rng = np.random.default_rng(4)
    q, kv, _ = rand_inputs(rng, 2, 2, 4, 6, 4)
    q *= 40.0                                           # logits of order +-hundreds
    idx = np.array([[0, 1, 2, 3], [3, -1, -1, -1]])
    _, lse = sparse_mla_fwd(q, kv, idx, 1.0, d_v=4)
    for s in range(2):
        J = idx[s][idx[s] != -1]
        ref = torch.logsumexp(torch.tensor(q[s] @ kv[J].T), dim=-1).numpy()
        np.testing.assert_allclose(lse[s], ref, rtol=1e-14, atol=1e-12)
