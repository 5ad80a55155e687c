"""Pins of the grouped (several KV groups) oracle, independent of its code:

  * brute force: per-(token, head) softmax attention written out with Python
    loops over a tiny grouped input, head h reading kv group h // (H / G) and
    index row idx[s, g] (a wrong head-to-group map, e.g. h % G, fails);
  * G = 1 is the single-group oracle exactly;
  * relabelling the groups (kv groups, index groups and head blocks together)
    relabels every output;
  * the backward is the gradient of the forward: central finite differences
    of sum(dout * out) along random directions in q and kv.
"""
import math

import numpy as np
import pytest

from oracle import (sparse_mla_bwd, sparse_mla_bwd_grouped, sparse_mla_fwd,
                    sparse_mla_fwd_grouped)
from oracle.smla_oracle import OracleInputError

DK, DV = 576, 512


def tiny(seed=0, S=3, H=4, G=2, K=3, S_kv=5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((S, H, DK)) * 0.3
    kv = rng.standard_normal((S_kv, G, DK)) * 0.3
    dout = rng.standard_normal((S, H, DV))
    idx = rng.integers(0, S_kv, size=(S, G, K)).astype(np.int32)
    idx[0, G - 1, 1] = -1      # padding inside a row
    idx[1, 0, :] = -1          # an empty row in group 0 only
    return q, kv, dout, idx


def brute_fwd(q, kv, idx, scale):
    S, H, _ = q.shape
    G = kv.shape[1]
    hg = H // G
    out = np.zeros((S, H, DV))
    lse = np.zeros((S, H))
    for s in range(S):
        for h in range(H):
            g = h // hg
            rows = [int(j) for j in idx[s, g] if j != -1]
            if not rows:
                lse[s, h] = math.log(1e-30)
                continue
            z = [scale * sum(q[s, h, d] * kv[j, g, d] for d in range(DK)) for j in rows]
            m = max(z)
            tot = sum(math.exp(v - m) for v in z)
            lse[s, h] = m + math.log(tot)
            for k, j in enumerate(rows):
                out[s, h] += math.exp(z[k] - lse[s, h]) * kv[j, g, :DV]
    return out, lse


def test_brute_force_forward():
    q, kv, dout, idx = tiny()
    out, lse = sparse_mla_fwd_grouped(q, kv, idx, 0.07)
    b_out, b_lse = brute_fwd(q, kv, idx, 0.07)
    np.testing.assert_allclose(out, b_out, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, b_lse, rtol=1e-12, atol=1e-12)
    assert np.all(out[1, :2] == 0.0) and np.all(out[1, 2:] != 0.0)


def test_one_group_is_the_single_group_oracle():
    q, kv, dout, idx = tiny(seed=1, G=1, H=3)
    out, lse = sparse_mla_fwd_grouped(q, kv, idx, 0.05)
    r_out, r_lse = sparse_mla_fwd(q, kv[:, 0], idx[:, 0], 0.05)
    assert np.array_equal(out, r_out) and np.array_equal(lse, r_lse)
    dq, dkv = sparse_mla_bwd_grouped(q, kv, dout, idx, 0.05)
    r_dq, r_dkv = sparse_mla_bwd(q, kv[:, 0], dout, idx[:, 0], 0.05)
    assert np.array_equal(dq, r_dq) and np.array_equal(dkv[:, 0], r_dkv)


def test_relabelling_groups_relabels_outputs():
    q, kv, dout, idx = tiny(seed=2, S=4, H=6, G=3, K=4, S_kv=6)
    perm = [2, 0, 1]
    hp = np.concatenate([np.arange(2 * g, 2 * g + 2) for g in perm])
    out, lse = sparse_mla_fwd_grouped(q, kv, idx, 0.1)
    dq, dkv = sparse_mla_bwd_grouped(q, kv, dout, idx, 0.1)
    p_out, p_lse = sparse_mla_fwd_grouped(q[:, hp], kv[:, perm], idx[:, perm], 0.1)
    p_dq, p_dkv = sparse_mla_bwd_grouped(q[:, hp], kv[:, perm], dout[:, hp], idx[:, perm], 0.1)
    assert np.array_equal(p_out, out[:, hp]) and np.array_equal(p_lse, lse[:, hp])
    assert np.array_equal(p_dq, dq[:, hp]) and np.array_equal(p_dkv, dkv[:, perm])


def test_backward_is_the_gradient_of_the_forward():
    q, kv, dout, idx = tiny(seed=3)
    scale = 0.08
    dq, dkv = sparse_mla_bwd_grouped(q, kv, dout, idx, scale)
    rng = np.random.default_rng(4)

    def loss(qq, kk):
        return float((sparse_mla_fwd_grouped(qq, kk, idx, scale)[0] * dout).sum())

    eps = 1e-5
    for _ in range(3):
        dqd = rng.standard_normal(q.shape)
        dkd = rng.standard_normal(kv.shape)
        fd_q = (loss(q + eps * dqd, kv) - loss(q - eps * dqd, kv)) / (2 * eps)
        fd_k = (loss(q, kv + eps * dkd) - loss(q, kv - eps * dkd)) / (2 * eps)
        assert fd_q == pytest.approx(float((dq * dqd).sum()), rel=1e-6, abs=1e-9)
        assert fd_k == pytest.approx(float((dkv * dkd).sum()), rel=1e-6, abs=1e-9)


def test_heads_must_split_over_groups():
    q, kv, dout, idx = tiny(seed=5, H=3, G=2)
    with pytest.raises(OracleInputError):
        sparse_mla_fwd_grouped(q, kv, idx, 0.1)
