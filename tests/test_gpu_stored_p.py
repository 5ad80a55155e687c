"""GPU parity of the stored-P backward (SMLA_DKV_STORED_P: the dq pass stores
P and scale * dS per union entry and query row, the dkv pass reads them
instead of recomputing the scores and dP): dq is bit for bit the recomputing
mode's (the dq pass only adds stores), dkv matches the oracle given the same
out / lse within the tolerance, rows no slot selects stay exact zeros (and
keep a -0.0 sign bit when accumulating), the result is bitwise reproducible,
and it composes with the atomic dkv mode and with the plan built once.
Workloads cover padding anywhere, empty rows, repeated indices, several kv
blocks per group, kv spans beyond one planner window and H = 8..128."""
import numpy as np
import pytest

from oracle import sparse_mla_bwd as o_bwd, touched_rows
from tests.helpers import TOL, bf16_to_np64, gpu_inputs, oracle_inputs, rel_err
from workloads import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES = {
    "tiny": synth.tiny,
    "ragged_dups_h16": lambda: synth.custom(S=70, H=16, K=96, S_kv=300, seed=21, dup_frac=0.1,
                                            pad_frac=0.2, empty_frac=0.05),
    "multi_block_h8": lambda: synth.custom(S=96, H=8, K=512, S_kv=1500, seed=22, pad_frac=0.1),
    "h32": lambda: synth.custom(S=40, H=32, K=200, S_kv=900, seed=23, pad_frac=0.3),
    "h64": lambda: synth.custom(S=33, H=64, K=130, S_kv=700, seed=24, pad_frac=0.25, dup_frac=0.05),
    "h128": lambda: synth.custom(S=21, H=128, K=150, S_kv=500, seed=26, pad_frac=0.2,
                                 empty_frac=0.1),
    "max_topk": lambda: synth.custom(S=16, H=8, K=16384, S_kv=20000, seed=27, pad_frac=0.2,
                                     empty_frac=0.0, dup_frac=0.05),
    "windows": lambda: synth.custom(S=12, H=16, K=700, S_kv=40000, seed=9, pad_frac=0.2,
                                    empty_frac=0.0),
    "oob": lambda: synth.custom(S=50, H=8, K=64, S_kv=200, seed=25, oob_frac=0.05),
}


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bwd_sparse_mla_amd
    bwd_sparse_mla_amd.load_library()


@pytest.mark.parametrize("case", list(CASES))
def test_stored_p_matches_oracle_and_recompute(case):
    import bwd_sparse_mla_amd as smla
    w = CASES[case]()
    print(f"[stored-p] {case} S={w.S} H={w.H} K={w.K} S_kv={w.S_kv}", flush=True)
    q, kv, dout, idx = gpu_inputs(w)
    out, lse = smla.sparse_mla_fwd(q, kv, idx, w.sm_scale)
    dq_r, dkv_r = smla.sparse_mla_bwd(q, kv, out, dout, idx, lse, w.sm_scale)
    dq_s, dkv_s = smla.sparse_mla_bwd(q, kv, out, dout, idx, lse, w.sm_scale, stored_p=True)
    dq_t, dkv_t = smla.sparse_mla_bwd(q, kv, out, dout, idx, lse, w.sm_scale, stored_p=True)
    torch.cuda.synchronize()
    assert torch.equal(dq_s.view(torch.int16), dq_r.view(torch.int16))
    assert torch.equal(dkv_s.view(torch.int16), dkv_t.view(torch.int16)), "not reproducible"
    assert torch.isfinite(dkv_s.float()).all()
    valid = (w.idx >= 0) & (w.idx < w.S_kv)
    oidx = np.where(valid, w.idx, -1).astype(np.int32)
    q64, kv64, do64 = oracle_inputs(w)
    _, s_dkv = o_bwd(q64, kv64, do64, oidx, w.sm_scale, out=bf16_to_np64(out),
                     lse=lse.cpu().numpy().astype(np.float64))
    g = bf16_to_np64(dkv_s)
    err, err_r = rel_err(g, s_dkv), rel_err(bf16_to_np64(dkv_r), s_dkv)
    print(f"[stored-p] {case} dkv rel error {err:.3e} (recomputing mode {err_r:.3e})", flush=True)
    assert err <= TOL
    untouched = ~touched_rows(oidx, w.S_kv)
    assert np.all(g[untouched] == 0.0)


@pytest.mark.parametrize("case", ["ragged_dups_h16", "multi_block_h8"])
def test_stored_p_atomic_and_accumulate(case):
    import bwd_sparse_mla_amd as smla
    w = CASES[case]()
    print(f"[stored-p] atomic / accumulate {case}", flush=True)
    q, kv, dout, idx = gpu_inputs(w)
    out, lse = smla.sparse_mla_fwd(q, kv, idx, w.sm_scale)
    d32 = torch.empty(w.S_kv, 576, dtype=torch.float32, device="cuda")
    smla.sparse_mla_bwd(q, kv, out, dout, idx, lse, w.sm_scale, dkv_f32=d32, stored_p=True)
    a32 = torch.empty(w.S_kv, 576, dtype=torch.float32, device="cuda")
    smla.sparse_mla_bwd(q, kv, out, dout, idx, lse, w.sm_scale, dkv_f32=a32, stored_p=True,
                        atomic=True)
    acc = torch.full((w.S_kv, 576), -0.0, dtype=torch.float32, device="cuda")
    smla.sparse_mla_bwd(q, kv, out, dout, idx, lse, w.sm_scale, dkv_f32=acc, accumulate=True,
                        stored_p=True)
    torch.cuda.synchronize()
    scale = float(d32.abs().max())
    assert float((a32 - d32).abs().max()) <= 1e-5 * max(scale, 1e-30)
    touched = touched_rows(w.idx, w.S_kv)
    bits = acc.view(torch.int32).cpu().numpy()
    assert np.array_equal(np.all(bits == np.int32(-2 ** 31), axis=1), ~touched)
    t = torch.from_numpy(touched).cuda()
    assert torch.equal(acc[t], d32[t])


def test_stored_p_with_the_plan_built_once():
    import bwd_sparse_mla_amd as smla
    w = CASES["multi_block_h8"]()
    print("[stored-p] plan once", flush=True)
    q, kv, dout, idx = gpu_inputs(w)
    run = smla.SparseMLARunner(w.S, w.S_kv, w.H, w.K, q.device, dkv_stored_p=True)
    run.plan(idx)
    run.fwd(q, kv, idx, w.sm_scale, planned=True)
    dq, dkv = run.bwd(q, kv, dout, idx, w.sm_scale, planned=True)
    out, lse = smla.sparse_mla_fwd(q, kv, idx, w.sm_scale)
    dq_s, dkv_s = smla.sparse_mla_bwd(q, kv, out, dout, idx, lse, w.sm_scale, stored_p=True)
    torch.cuda.synchronize()
    assert torch.equal(dq.view(torch.int16), dq_s.view(torch.int16))
    assert torch.equal(dkv.view(torch.int16), dkv_s.view(torch.int16))


@pytest.mark.parametrize("atomic", [False, True])
def test_stored_p_empty_query_batch(atomic):
    """No query rows: no dq launch builds the chunk lists, the schedule kernel
    runs on its own, and dkv is all zeros (kv blocks of an odd count)."""
    import bwd_sparse_mla_amd as smla
    w = synth.custom(S=4, H=8, K=4, S_kv=70, seed=15)
    print(f"[stored-p] empty batch atomic={atomic}", flush=True)
    q, kv, dout, idx = gpu_inputs(w)
    out, lse = smla.sparse_mla_fwd(q[:0], kv, idx[:0], w.sm_scale)
    d32 = torch.full((w.S_kv, 576), 7.0, dtype=torch.float32, device="cuda")
    dq, dkv = smla.sparse_mla_bwd(q[:0], kv, out, dout[:0], idx[:0], lse, w.sm_scale, dkv_f32=d32,
                                  stored_p=True, atomic=atomic)
    torch.cuda.synchronize()
    assert dq.shape == (0, 8, 576)
    assert torch.count_nonzero(dkv).item() == 0 and torch.count_nonzero(d32).item() == 0
