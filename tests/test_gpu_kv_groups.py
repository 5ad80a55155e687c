"""GPU parity with several KV groups (kv [S_kv, G, 576], indices [S, G, K];
head block g of H / G heads attends over kv group g): forward against the
grouped oracle; backward (deterministic, stored-P, atomic dkv) against the
grouped oracle given the GPU's out / lse; rows of a group no slot selects stay
exact zeros in dkv; empty index rows give zero out and dq; the plan built once
gives the one-shot results bit for bit.  Cases cover 8 to 128 heads per group
(below 64 the kernels walk the (token, group) pairs in group-major order),
kv blocks that straddle two groups, more than 16384 flat kv rows, padding
anywhere, empty rows, repeated and out-of-range indices, index rows that are
not a multiple of 16 bytes."""
import numpy as np
import pytest

from oracle import sparse_mla_bwd_grouped, sparse_mla_fwd_grouped
from tests.helpers import TOL, bf16_to_np64, rel_err, to_torch_bf16
from workloads import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES = {
    "h16_g2": dict(S=37, H=16, G=2, K=120, S_kv=300, seed=41, pad_frac=0.3, empty_frac=0.1),
    "h32_g4_dups": dict(S=20, H=32, G=4, K=200, S_kv=500, seed=42, pad_frac=0.2, dup_frac=0.1),
    "h64_g8_oob": dict(S=25, H=64, G=8, K=64, S_kv=90, seed=43, pad_frac=0.2, oob_frac=0.05),
    "h256_g2": dict(S=9, H=256, G=2, K=100, S_kv=200, seed=44, pad_frac=0.25, empty_frac=0.1),
    "h128_g2_multiblock": dict(S=30, H=128, G=2, K=400, S_kv=1200, seed=45, pad_frac=0.1),
    # index rows of 600 bytes (K not a multiple of 4), read where the caller keeps them
    "h32_g2_k150": dict(S=23, H=32, G=2, K=150, S_kv=400, seed=46, pad_frac=0.2, empty_frac=0.1),
    # three tokens, 8 heads per group: one 64-row query group spans three kv groups
    "h64_g8_s3_dups": dict(S=3, H=64, G=8, K=50, S_kv=70, seed=47, pad_frac=0.2, dup_frac=0.1),
    # more than 16384 flat kv rows (the planner scans each group's span; the
    # query group of pairs 32..39 holds both kv groups' rows: two windows)
    "h16_g2_wide": dict(S=37, H=16, G=2, K=300, S_kv=9000, seed=48, pad_frac=0.2, dup_frac=0.02),
    # 64 heads per group (token-major pairs), 20000 flat kv rows
    "h256_g4_wide": dict(S=6, H=256, G=4, K=200, S_kv=5000, seed=49, pad_frac=0.2),
}


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bwd_sparse_mla_amd
    bwd_sparse_mla_amd.load_library()


def _inputs(w):
    return (to_torch_bf16(w.q), to_torch_bf16(w.kv), to_torch_bf16(w.dout),
            torch.from_numpy(np.ascontiguousarray(w.idx)).cuda())


def _clean(idx, s_kv):
    return np.where((idx >= 0) & (idx < s_kv), idx, -1).astype(np.int32)


@pytest.mark.parametrize("case", list(CASES))
def test_kv_groups_match_the_grouped_oracle(case):
    import bwd_sparse_mla_amd as smla
    w = synth.custom_grouped(**CASES[case])
    print(f"[kv-groups] {case} S={w.S} H={w.H} G={w.G} K={w.K} S_kv={w.S_kv}", flush=True)
    q, kv, dout, idx = _inputs(w)
    out, lse = smla.sparse_mla_fwd(q, kv, idx, w.sm_scale)
    res = {}
    for mode in ("deterministic", "stored", "atomic"):
        res[mode] = smla.sparse_mla_bwd(q, kv, out, dout, idx, lse, w.sm_scale,
                                        stored_p=mode == "stored", atomic=mode == "atomic")
    torch.cuda.synchronize()
    oidx = _clean(w.idx, w.S_kv)
    q64, kv64, do64 = (synth.bf16_bits_to_f64(a) for a in (w.q, w.kv, w.dout))
    r_out, r_lse = sparse_mla_fwd_grouped(q64, kv64, oidx, w.sm_scale)
    g_out, g_lse = bf16_to_np64(out), lse.cpu().numpy().astype(np.float64)
    s_dq, s_dkv = sparse_mla_bwd_grouped(q64, kv64, do64, oidx, w.sm_scale, out=g_out, lse=g_lse)
    errs = {"out": rel_err(g_out, r_out), "lse": rel_err(g_lse, r_lse)}
    for mode, (dq, dkv) in res.items():
        errs[f"dq/{mode}"] = rel_err(bf16_to_np64(dq), s_dq)
        errs[f"dkv/{mode}"] = rel_err(bf16_to_np64(dkv), s_dkv)
    print(f"[kv-groups] {case} rel errors {errs}", flush=True)
    for k, v in errs.items():
        assert v <= TOL, f"{k} relative error {v:.3e} > {TOL}"
    assert torch.equal(res["stored"][0].view(torch.int16), res["deterministic"][0].view(torch.int16))
    # rows of a group that no slot of that group selects: exact zeros
    for g in range(w.G):
        touched = np.zeros(w.S_kv, dtype=bool)
        v = oidx[:, g][oidx[:, g] >= 0]
        touched[v] = True
        for mode, (dq, dkv) in res.items():
            d = dkv[:, g].float().cpu().numpy()
            assert np.all(d[~touched] == 0.0), f"group {g} {mode}: dkv on unselected rows"
        hg = w.H // w.G
        empty = ~(oidx[:, g] >= 0).any(axis=1)
        if empty.any():
            e = torch.as_tensor(np.nonzero(empty)[0], device="cuda")
            assert float(out.index_select(0, e)[:, g * hg:(g + 1) * hg].float().abs().sum()) == 0.0
            dq = res["deterministic"][0]
            assert float(dq.index_select(0, e)[:, g * hg:(g + 1) * hg].float().abs().sum()) == 0.0


def test_kv_groups_with_the_plan_built_once():
    import bwd_sparse_mla_amd as smla
    w = synth.custom_grouped(**CASES["h32_g4_dups"])
    print("[kv-groups] plan once", flush=True)
    q, kv, dout, idx = _inputs(w)
    run = smla.SparseMLARunner(w.S, w.S_kv, w.H, w.K, q.device, dkv_stored_p=True,
                               kv_groups=w.G)
    run._check(q, kv, idx, dout)
    run.plan(idx)
    run.fwd(q, kv, idx, w.sm_scale, planned=True)
    dq, dkv = run.bwd(q, kv, dout, idx, w.sm_scale, planned=True)
    out, lse = smla.sparse_mla_fwd(q, kv, idx, w.sm_scale)
    dq1, dkv1 = smla.sparse_mla_bwd(q, kv, out, dout, idx, lse, w.sm_scale, stored_p=True)
    torch.cuda.synchronize()
    assert torch.equal(run.out.view(torch.int16), out.view(torch.int16))
    assert torch.equal(dq.view(torch.int16), dq1.view(torch.int16))
    assert torch.equal(dkv.view(torch.int16), dkv1.view(torch.int16))
