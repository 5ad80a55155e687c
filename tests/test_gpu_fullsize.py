"""Parity at the full sizes of the four large workloads, in the launch
configuration bench.py times (SparseMLARunner: every buffer preallocated, the
index plan built once, one forward and one backward call on it).

At the two H = 8 workloads (packed ragged batch, padding stress) the oracle
covers every token in seconds, so out, lse, dq and dkv are compared over
whole tensors.  At the larger ones (recency, long context, 128 heads) the
oracle checks sampled outputs it computes one by one, and the rest is held to
properties that hold at any size:

  * out / lse / dq of sampled tokens (first and last token of every sequence,
    empty rows, random tokens) against the oracle's forward and its backward
    given the GPU's out / lse;
  * dkv of sampled kv rows against the oracle's sum over every token that
    selects them (rows chosen so that the selecting tokens stay few);
  * exact zeros: out, dq of all-padding rows, and dkv of every kv row no slot
    selects (bit-exact index handling over the whole tensor);
  * no NaN / Inf anywhere.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

from oracle import sparse_mla_bwd as o_bwd
from oracle import sparse_mla_fwd as o_fwd
from tests.helpers import TOL, gpu_inputs, rel_err
from workloads import synth

pytestmark = pytest.mark.gpu

MAX_SELECTORS = 768   # tokens the oracle recomputes for the sampled dkv rows


def _run(w, atomic=False, stored=False):
    import torch

    import bwd_sparse_mla_amd as smla
    q, kv, dout, idx = gpu_inputs(w)
    run = smla.SparseMLARunner(w.S, w.S_kv, w.H, w.K, q.device, dkv_atomic=atomic,
                               dkv_stored_p=stored)
    run._check(q, kv, idx, dout)
    run.plan(idx)
    run.fwd(q, kv, idx, w.sm_scale, planned=True)
    run.bwd(q, kv, dout, idx, w.sm_scale, planned=True)
    torch.cuda.synchronize()
    return run


def _tokens(w, rng, n_random=16):
    starts = np.concatenate([[0], np.cumsum(w.seqlens)[:-1]])
    ends = np.cumsum(w.seqlens) - 1
    valid = (w.idx >= 0) & (w.idx < w.S_kv)
    empty = np.nonzero(~valid.any(axis=1))[0]
    picks = list(starts) + list(ends) + list(empty[:4])
    picks += list(rng.choice(w.S, size=n_random, replace=False))
    return np.unique(np.asarray(picks, dtype=np.int64))


def _rows(w, rng):
    """kv rows near the end of each sequence (selected by few tokens) plus a
    few random ones, kept while the selecting tokens stay within budget."""
    ends = np.cumsum(w.seqlens) - 1
    cand = [e - d for e in ends for d in (0, 3, 17)]
    cand += list(rng.choice(w.S_kv, size=8, replace=False))
    rows, sel = [], np.zeros(w.S, dtype=bool)
    for j in cand:
        hits = (w.idx == j).any(axis=1)
        if (sel | hits).sum() > MAX_SELECTORS:
            continue
        rows.append(int(j))
        sel |= hits
    return np.asarray(sorted(set(rows)), dtype=np.int64), np.nonzero(sel)[0]


def _bf16_rows(t, rows):
    import torch
    return t.index_select(0, torch.as_tensor(rows, device=t.device)).float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name,atomic,stored", [
    ("packed_ragged", False, False), ("padding_stress", False, False), ("recency", False, False),
    ("long_context", False, False), ("long_context", True, False),
    ("packed_ragged", False, True), ("padding_stress", False, True), ("recency", False, True),
    ("long_context", True, True), ("heads128", False, False), ("heads128", False, True)])
def test_full_size_sampled_parity(name, atomic, stored):
    """atomic: the same checks with dkv scattered by fp32 atomic adds (the
    long-context workload runs in both dkv modes); stored: the dkv pass reads
    P and dS stored by the dq pass instead of recomputing them."""
    import torch

    w = synth.WORKLOADS[name]()
    print(f"[fullsize] {w.name} S={w.S} H={w.H} K={w.K} S_kv={w.S_kv} valid={w.n_valid} "
          f"dkv {'atomic' if atomic else 'deterministic'} "
          f"{'stored P' if stored else 'recomputed P'}", flush=True)
    run = _run(w, atomic, stored)
    for label, t in (("out", run.out), ("lse", run.lse), ("dq", run.dq), ("dkv", run.dkv)):
        bad = int((~torch.isfinite(t.float())).sum())
        assert bad == 0, f"{bad} nonfinite values in {label}"

    rng = np.random.default_rng(99)
    toks = _tokens(w, rng)
    rows, selectors = _rows(w, rng)
    sub = np.union1d(toks, selectors)                     # tokens the oracle needs
    pos = np.searchsorted(sub, toks)                      # sampled tokens inside sub

    kv64 = synth.bf16_bits_to_f64(w.kv)
    q64 = synth.bf16_bits_to_f64(w.q[sub])
    do64 = synth.bf16_bits_to_f64(w.dout[sub])
    ix = w.idx[sub]
    g_out = _bf16_rows(run.out, sub)
    g_lse = run.lse.index_select(0, torch.as_tensor(sub, device=run.lse.device)).cpu().numpy().astype(np.float64)
    g_dq = _bf16_rows(run.dq, toks)
    g_dkv = _bf16_rows(run.dkv, rows)

    r_out, r_lse = o_fwd(q64, kv64, ix, w.sm_scale, tokens=pos)
    s_dq, s_dkv = o_bwd(q64, kv64, do64, ix, w.sm_scale, out=g_out, lse=g_lse, tokens=pos,
                        rows=rows)
    errs = {"out": rel_err(g_out[pos], r_out), "lse": rel_err(g_lse[pos], r_lse),
            "dq": rel_err(g_dq, s_dq), "dkv": rel_err(g_dkv, s_dkv)}
    print(f"[fullsize] {w.name} tokens={len(toks)} rows={len(rows)} selectors={len(selectors)} "
          f"rel errors {errs}", flush=True)
    for k, v in errs.items():
        assert v <= TOL, f"{k} relative error {v:.3e} > {TOL} on sampled outputs"

    # all-padding rows: exact zeros and the floor's LSE
    valid = (w.idx >= 0) & (w.idx < w.S_kv)
    empty = np.nonzero(~valid.any(axis=1))[0]
    if empty.size:
        e = torch.as_tensor(empty, device=run.out.device)
        assert float(run.out.index_select(0, e).float().abs().sum()) == 0.0
        assert float(run.dq.index_select(0, e).float().abs().sum()) == 0.0
        le = run.lse.index_select(0, e).cpu().numpy()
        assert np.allclose(le, math.log(1e-30), rtol=1e-6, atol=0)

    # bit-exact index handling: dkv rows no slot selects are exactly +0
    touched = np.zeros(w.S_kv, dtype=bool)
    touched[w.idx[valid]] = True
    bits = run.dkv.view(torch.int16).cpu().numpy()
    assert not bits[~touched].any(), "dkv written on a row no slot selects"
    nonzero_rows = bits.any(axis=1)
    assert nonzero_rows.sum() == touched.sum(), "a selected kv row got no gradient"


@pytest.mark.parametrize("name", ["packed_ragged", "padding_stress"])
def test_full_size_whole_tensor_parity(name):
    """Element-by-element parity over whole tensors at the two H = 8 workloads
    (the oracle covers all 4096 tokens in seconds): out, lse against its
    forward; dq, dkv of both backward forms against its backward given the
    GPU's out / lse; the end-to-end error (gradient recomputed from scratch)
    is printed, and gated at unit variance."""
    import torch

    w = synth.WORKLOADS[name]()
    print(f"[fullsize-whole] {w.name} S={w.S} H={w.H} K={w.K} valid={w.n_valid}", flush=True)
    runs = {stored: _run(w, stored=stored) for stored in (False, True)}
    base = runs[True]
    assert torch.equal(runs[False].out, base.out) and torch.equal(runs[False].lse, base.lse)
    kv64 = synth.bf16_bits_to_f64(w.kv)
    q64 = synth.bf16_bits_to_f64(w.q)
    do64 = synth.bf16_bits_to_f64(w.dout)
    g_out = base.out.float().cpu().numpy().astype(np.float64)
    g_lse = base.lse.cpu().numpy().astype(np.float64)
    r_out, r_lse = o_fwd(q64, kv64, w.idx, w.sm_scale)
    s_dq, s_dkv = o_bwd(q64, kv64, do64, w.idx, w.sm_scale, out=g_out, lse=g_lse)
    e_dq, e_dkv = o_bwd(q64, kv64, do64, w.idx, w.sm_scale)
    errs = {"out": rel_err(g_out, r_out), "lse": rel_err(g_lse, r_lse)}
    assert np.isfinite(g_out).all() and np.isfinite(g_lse).all()
    for stored, run in runs.items():
        g_dq = run.dq.float().cpu().numpy().astype(np.float64)
        g_dkv = run.dkv.float().cpu().numpy().astype(np.float64)
        assert np.isfinite(g_dq).all() and np.isfinite(g_dkv).all()
        tag = "stored" if stored else "recompute"
        errs[f"dq_{tag}"] = rel_err(g_dq, s_dq)
        errs[f"dkv_{tag}"] = rel_err(g_dkv, s_dkv)
        e2e = {"dq": rel_err(g_dq, e_dq), "dkv": rel_err(g_dkv, e_dkv)}
        print(f"[fullsize-whole] {w.name} {tag}: end-to-end {e2e}", flush=True)
        if name == "packed_ragged":    # unit variance: the end-to-end gate holds too
            for k, v in e2e.items():
                assert v <= TOL, f"end-to-end {k} ({tag}) relative error {v:.3e}"
    print(f"[fullsize-whole] {w.name} rel errors {errs}", flush=True)
    for k, v in errs.items():
        assert v <= TOL, f"{k} relative error {v:.3e} > {TOL} over the whole tensor"
