"""smla_fwd_noalloc (the forward with the library's fixed per-device scratch
buffer instead of a caller's workspace) against smla_fwd, through the C ABI:
bit for bit on two calls in a row, the second with a smaller input (the
scratch keeps the first call's contents), and the second also against the
oracle."""
import ctypes

import numpy as np
import pytest

from oracle import sparse_mla_fwd as o_fwd
from tests.helpers import TOL, bf16_to_np64, gpu_inputs, oracle_inputs, rel_err
from workloads import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def run_both(lib, w):
    """(out, lse) from smla_fwd with a fresh workspace and from
    smla_fwd_noalloc, same inputs, same stream."""
    from bwd_sparse_mla_amd import _lib
    q, kv, _, idx = gpu_inputs(w)
    S, H, K, S_kv = w.S, w.H, w.K, w.S_kv
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    outs = []
    for noalloc in (False, True):
        out = torch.full((S, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((S, H), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            st = lib.smla_fwd_noalloc(_p(q), _p(kv), _p(idx), S, S_kv, H, K, float(w.sm_scale),
                                      _p(out), _p(lse), stream)
        else:
            nbytes = lib.smla_fwd_workspace_size(S, S_kv, H, K)
            ws = torch.empty(nbytes + 256, dtype=torch.uint8, device="cuda")
            addr = (ws.data_ptr() + 255) & ~255
            st = lib.smla_fwd(_p(q), _p(kv), _p(idx), S, S_kv, H, K, float(w.sm_scale), _p(out),
                              _p(lse), ctypes.c_void_p(addr), nbytes, stream)
        _lib.check(st)
        torch.cuda.synchronize()
        outs.append((out, lse))
    return outs


def test_noalloc_forward_matches_the_workspace_forward_twice():
    from bwd_sparse_mla_amd import _lib
    lib = _lib.load()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    big = synth.packed_ragged()     # 42 MB of the 64 MiB scratch
    small = synth.custom(S=37, H=8, K=300, S_kv=333, seed=61, pad_frac=0.4, empty_frac=0.1)
    for w in (big, small):
        print(f"[noalloc] {w.name} S={w.S} H={w.H} K={w.K} S_kv={w.S_kv}", flush=True)
        (o_ref, l_ref), (o_na, l_na) = run_both(lib, w)
        assert torch.equal(o_ref.view(torch.int16), o_na.view(torch.int16)), w.name
        assert torch.equal(l_ref.view(torch.int32), l_na.view(torch.int32)), w.name
    # the second (smaller) call against the oracle
    q64, kv64, _ = oracle_inputs(small)
    r_out, r_lse = o_fwd(q64, kv64, small.idx, small.sm_scale)
    errs = {"out": rel_err(bf16_to_np64(o_na), r_out),
            "lse": rel_err(l_na.cpu().numpy().astype(np.float64), r_lse)}
    print(f"[noalloc] {small.name} rel errors {errs}", flush=True)
    assert max(errs.values()) <= TOL


def test_noalloc_refuses_a_shape_beyond_the_scratch_on_the_device():
    from bwd_sparse_mla_amd import _lib
    lib = _lib.load()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S, H, K, S_kv = 8192, 16, 2048, 8192
    out = torch.zeros(1, dtype=torch.bfloat16, device="cuda")
    st = lib.smla_fwd_noalloc(_p(out), _p(out), _p(out), S, S_kv, H, K, 0.1, _p(out), _p(out),
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert _lib.STATUS_NAMES[st] == "SMLA_ERR_WORKSPACE"
    assert "smla_fwd_noalloc" in lib.smla_last_error().decode()
