"""Plant plausible mistakes into a copy of the oracle (on the CPU) and check
that the pins catch every one: a dropped term, a wrong sign, a wrong index or
slice, a transposed or mis-reduced operand, a missing scale."""
import importlib.util
import math
import os
import types

import numpy as np
import pytest

from tests.test_oracle_pins import (causal_full_idx, dense_causal_torch,
                                    gather_autograd_torch, rand_inputs,
                                    supplied_lse_shift_ok, supplied_out_perturbation_ok)

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "smla_oracle.py")

MUTATIONS = {
    "rope_tail_dropped_from_scores": ("z = scale * (q_s @ rows.T)",
                                      "z = scale * (q_s @ rows[:, :d_v].T)"),
    "dS_sign_flipped": ("ds = p * (dp - delta[:, None])", "ds = p * (dp + delta[:, None])"),
    "delta_dropped": ("ds = p * (dp - delta[:, None])", "ds = p * dp"),
    "dV_term_dropped": ("contrib[:, :d_v] += p.T @ dout_s", "contrib[:, :d_v] += 0.0"),
    "dq_scale_missing": ("dq_s = scale * (ds @ rows)", "dq_s = (ds @ rows)"),
    "dk_scale_missing": ("contrib = scale * (ds.T @ q_s)", "contrib = (ds.T @ q_s)"),
    "value_slice_shifted": ("out = p @ rows[:, :d_v]", "out = p @ rows[:, 1:d_v + 1]"),
    "row_zero_treated_as_padding": ("keep = row != -1", "keep = row > 0"),
    "delta_mean_not_sum": ("delta = (dout_s * out_s).sum(axis=1)",
                           "delta = (dout_s * out_s).mean(axis=1)"),
    "lse_missing_max": ("lse = m + np.log(np.maximum(l, SUMEXP_FLOOR))",
                        "lse = np.log(np.maximum(l, SUMEXP_FLOOR))"),
    "dp_uses_keys_tail_shift": ("dp = dout_s @ rows[:, :d_v].T",
                                "dp = dout_s @ rows[:, -d_v:].T"),
    "duplicates_collapsed": ("np.add.at(dkv, J, contrib)", "dkv[J] += contrib"),
    # the supplied-out / lse branch (the backward call takes the forward's
    # saved out and lse)
    "supplied_lse_ignored": ("p = np.exp(z - lse[s][:, None])",
                             "p = token_forward(q[s], R, sm_scale, d_v)[2]"),
    "supplied_out_ignored": ("o = out[s]", "o = token_forward(q[s], R, sm_scale, d_v)[0]"),
    "supplied_lse_base2": ("p = np.exp(z - lse[s][:, None])",
                           "p = np.exp2(z - lse[s][:, None])"),
}


def load_mutant(old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, old
    text = text.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(text, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def pins_pass(mod) -> bool:
    """The subset of pins the mutants are checked against."""
    rng = np.random.default_rng(31)
    # dense causal reduction (small dims so value slices matter)
    seqlens, H, K, DK, DV = [5, 4], 2, 6, 12, 8
    S = sum(seqlens)
    q, kv, dout = rand_inputs(rng, S, H, S, DK, DV)
    idx = causal_full_idx(rng, seqlens, K)
    try:
        out, lse = mod.sparse_mla_fwd(q, kv, idx, 0.5, d_v=DV)
        dq, dkv = mod.sparse_mla_bwd(q, kv, dout, idx, 0.5, d_v=DV)
    except Exception:
        return False
    r = dense_causal_torch(q, kv, dout, seqlens, 0.5, DV)
    for a, b in zip((out, lse, dq, dkv), r):
        if not np.allclose(a, b, rtol=1e-10, atol=1e-11):
            return False
    # brute force with padding and duplicates
    S, S_kv = 8, 6
    q, kv, dout = rand_inputs(rng, S, H, S_kv, DK, DV)
    idx = rng.integers(0, S_kv, size=(S, 7))
    idx[rng.random(idx.shape) < 0.3] = -1
    idx[:, 0] = 0                     # make sure row 0 is selected
    idx[1, 1:3] = idx[1, 0]           # a duplicate
    try:
        out, lse = mod.sparse_mla_fwd(q, kv, idx, 0.7, d_v=DV)
        dq, dkv = mod.sparse_mla_bwd(q, kv, dout, idx, 0.7, d_v=DV)
    except Exception:
        return False
    r_out, r_lse, r_dq, r_dkv = gather_autograd_torch(q, kv, dout, idx, 0.7, DV)
    ne = ~np.isnan(r_lse)
    # the supplied-out / lse branch away from its fixed point
    try:
        if not (supplied_lse_shift_ok(mod) and supplied_out_perturbation_ok(mod)):
            return False
    except Exception:
        return False
    return (np.allclose(out, r_out, rtol=1e-10, atol=1e-11)
            and np.allclose(lse[ne], r_lse[ne], rtol=1e-10, atol=1e-11)
            and np.allclose(dq, r_dq, rtol=1e-10, atol=1e-11)
            and np.allclose(dkv, r_dkv, rtol=1e-10, atol=1e-11))


def test_unmutated_copy_passes():
    text = open(SRC).read()
    mod = types.ModuleType("oracle_copy")
    exec(compile(text, "oracle_copy", "exec"), mod.__dict__)
    assert pins_pass(mod)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutant_is_caught(name):
    old, new = MUTATIONS[name]
    assert not pins_pass(load_mutant(old, new)), f"pins missed the planted mistake {name}"
