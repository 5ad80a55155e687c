"""Out-of-bounds write guards and repeated-run stress, through the C ABI.

The fourth NaN class on the pages is an out-of-bounds atomic write into dKV
(miles PR #2079 digest, "fix GLM-5 sparse-MLA kernel -1 index OOB and NaN
gradients", key code snippets of the backward and 实现拆解 item 3), and the
compiler-aliasing class was caught by repeated stress runs (miles PR #1642
report, "disable aggressive smem merge in sparse-MLA backward", 风险与影响).

Guards: every buffer the library writes -- out, lse, dq, dkv, dkv_f32 and the
workspace -- is a view into a larger allocation whose bytes before and after
hold a sentinel pattern; after the calls the guard bytes must be unchanged,
and the guarded results must equal those of a plain call bit for bit (every
mode but the atomic one, which is held to the deterministic mode's values
within fp32 rounding).  Ragged s_kv (not a multiple of 64), padding, empty
rows, out-of-range indices and repeats are in the inputs.

Stress: 50 backward calls in a row, each checked before the next (the first
failure ends the test): the deterministic forms bit for bit, the atomic form
within fp32-summation-order rounding of the deterministic one.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

from oracle import sparse_mla_bwd as o_bwd
from tests.helpers import TOL, bf16_to_np64, gpu_inputs, oracle_inputs, rel_err
from workloads import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GUARD = 4096        # bytes of sentinel on each side (a multiple of 256)
SENTINEL = 0xA5


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bwd_sparse_mla_amd
    bwd_sparse_mla_amd.load_library()


class Guarded:
    """nbytes of device memory between two GUARD-byte sentinel bands."""

    def __init__(self, nbytes: int, fill: torch.Tensor | None = None):
        self.nbytes = nbytes
        self.buf = torch.full((nbytes + 2 * GUARD,), SENTINEL, dtype=torch.uint8, device="cuda")
        self.base = self.buf.data_ptr() + GUARD
        assert self.base % 256 == 0
        if fill is not None:
            src = fill.contiguous().view(torch.uint8).reshape(-1)
            assert src.numel() == nbytes
            self.buf[GUARD:GUARD + nbytes].copy_(src)

    @property
    def ptr(self):
        return ctypes.c_void_p(self.base)

    def view(self, dtype, shape):
        return self.buf[GUARD:GUARD + self.nbytes].view(dtype).reshape(shape)

    def guards_intact(self) -> bool:
        lo = self.buf[:GUARD]
        hi = self.buf[GUARD + self.nbytes:]
        return bool((lo == SENTINEL).all()) and bool((hi == SENTINEL).all())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def guarded_step(q, kv, dout, idx, scale, G, flags, with_dkv=True, dkv32_init=None):
    """One forward and one backward through smla_fwd_g / smla_bwd_g with every
    written buffer (and both workspaces) guarded.  Returns the results as
    tensors and the list of buffers whose guards were overwritten."""
    from bwd_sparse_mla_amd import _lib
    lib = _lib.load()
    S, H = q.shape[0], q.shape[1]
    S_kv = kv.shape[0]
    K = idx.shape[-1]
    out = Guarded(S * H * 512 * 2)
    lse = Guarded(S * H * 4)
    dq = Guarded(S * H * 576 * 2)
    dkv = Guarded(S_kv * G * 576 * 2) if with_dkv else None
    d32 = None
    if dkv32_init is not None or not with_dkv or flags & _lib.SMLA_DKV_ACCUMULATE:
        d32 = Guarded(S_kv * G * 576 * 4, dkv32_init)
    fws = Guarded(lib.smla_fwd_workspace_size_g(S, S_kv, H, G, K))
    bws = Guarded(lib.smla_bwd_workspace_size_g(S, S_kv, H, G, K, flags))
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    _lib.check(lib.smla_fwd_g(P(q), P(kv), P(idx), S, S_kv, H, G, K, float(scale), out.ptr,
                              lse.ptr, 0, fws.ptr, fws.nbytes, _stream()))
    _lib.check(lib.smla_bwd_g(P(q), P(kv), out.ptr, P(dout), P(idx), lse.ptr, S, S_kv, H, G, K,
                              float(scale), dq.ptr, dkv.ptr if dkv else ctypes.c_void_p(0),
                              d32.ptr if d32 else ctypes.c_void_p(0), flags, bws.ptr, bws.nbytes,
                              _stream()))
    torch.cuda.synchronize()
    bufs = {"out": out, "lse": lse, "dq": dq, "dkv": dkv, "dkv_f32": d32, "fwd_ws": fws,
            "bwd_ws": bws}
    broken = [k for k, b in bufs.items() if b is not None and not b.guards_intact()]
    res = {"out": out.view(torch.bfloat16, (S, H, 512)).clone(),
           "lse": lse.view(torch.float32, (S, H)).clone(),
           "dq": dq.view(torch.bfloat16, (S, H, 576)).clone()}
    if dkv:
        res["dkv"] = dkv.view(torch.bfloat16, (S_kv * G, 576)).clone()
    if d32:
        res["dkv_f32"] = d32.view(torch.float32, (S_kv * G, 576)).clone()
    return res, broken


def plain_step(q, kv, dout, idx, scale, flags, dkv_f32=None):
    import bwd_sparse_mla_amd as smla
    from bwd_sparse_mla_amd import _lib
    out, lse = smla.sparse_mla_fwd(q, kv, idx, scale)
    dq, dkv = smla.sparse_mla_bwd(q, kv, out, dout, idx, lse, scale, dkv_f32=dkv_f32,
                                  accumulate=bool(flags & _lib.SMLA_DKV_ACCUMULATE),
                                  atomic=bool(flags & _lib.SMLA_DKV_ATOMIC),
                                  stored_p=bool(flags & _lib.SMLA_DKV_STORED_P))
    torch.cuda.synchronize()
    return out, lse, dq, dkv


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


CASES = {
    # ragged s_kv, padding anywhere, empty rows, out-of-range entries, repeats
    "h8_ragged_oob": dict(S=37, H=8, K=300, S_kv=333, seed=41, pad_frac=0.4, empty_frac=0.1,
                          oob_frac=0.05, dup_frac=0.05),
    "h16_tail_rows": dict(S=50, H=16, K=200, S_kv=130, seed=42, pad_frac=0.2, empty_frac=0.05,
                          oob_frac=0.02),
    "h64_padding_heavy": dict(S=9, H=64, K=256, S_kv=65, seed=43, pad_frac=0.9, empty_frac=0.2,
                              oob_frac=0.05),
    "h128_one_block": dict(S=5, H=128, K=64, S_kv=63, seed=44, pad_frac=0.3, empty_frac=0.0),
}
MODES = ["deterministic", "stored_p", "atomic", "atomic_stored_p", "accumulate",
         "fp32_only"]


def mode_flags(mode):
    from bwd_sparse_mla_amd import _lib
    return {"deterministic": 0, "stored_p": _lib.SMLA_DKV_STORED_P,
            "atomic": _lib.SMLA_DKV_ATOMIC,
            "atomic_stored_p": _lib.SMLA_DKV_ATOMIC | _lib.SMLA_DKV_STORED_P,
            "accumulate": _lib.SMLA_DKV_ACCUMULATE | _lib.SMLA_DKV_STORED_P,
            "fp32_only": _lib.SMLA_DKV_STORED_P}[mode]


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("mode", MODES)
def test_no_write_outside_any_buffer(case, mode):
    w = synth.custom(**CASES[case])
    print(f"[guards] {case} {mode} S={w.S} H={w.H} K={w.K} S_kv={w.S_kv}", flush=True)
    q, kv, dout, idx = gpu_inputs(w)
    flags = mode_flags(mode)
    init = None
    if mode == "accumulate":
        init = torch.full((w.S_kv, 576), -0.0, dtype=torch.float32, device="cuda")
    res, broken = guarded_step(q, kv, dout, idx, w.sm_scale, 1, flags,
                               with_dkv=(mode != "fp32_only"), dkv32_init=init)
    assert not broken, f"writes past the end of {broken}"

    # the guarded call computes what the plain call computes
    ref32 = torch.full((w.S_kv, 576), -0.0, dtype=torch.float32, device="cuda")
    out, lse, dq, dkv = plain_step(q, kv, dout, idx, w.sm_scale, flags, dkv_f32=ref32)
    assert torch.equal(bits(res["out"]), bits(out))
    assert torch.equal(bits(res["lse"]), bits(lse))
    assert torch.equal(bits(res["dq"]), bits(dq))
    if "atomic" in mode:
        det = torch.empty_like(ref32)
        plain_step(q, kv, dout, idx, w.sm_scale, 0, dkv_f32=det)
        scale = max(float(det.abs().max()), 1e-30)
        assert float((res["dkv"].float() - det.to(torch.bfloat16).float()).abs().max()) <= 1e-2 * scale
    elif "dkv" in res:
        assert torch.equal(bits(res["dkv"]), bits(dkv))
    if "dkv_f32" in res:
        assert torch.equal(bits(res["dkv_f32"]), bits(ref32))


def test_grouped_kv_no_write_outside_any_buffer():
    from bwd_sparse_mla_amd import _lib
    w = synth.custom_grouped(S=21, H=32, G=2, K=150, S_kv=99, seed=45, pad_frac=0.3,
                             empty_frac=0.1)
    print(f"[guards] kv groups G={w.G} S={w.S} H={w.H} K={w.K} S_kv={w.S_kv}", flush=True)
    q = torch.from_numpy(w.q.view(np.int16)).view(torch.bfloat16).cuda()
    kv = torch.from_numpy(w.kv.view(np.int16)).view(torch.bfloat16).cuda()
    dout = torch.from_numpy(w.dout.view(np.int16)).view(torch.bfloat16).cuda()
    idx = torch.from_numpy(np.ascontiguousarray(w.idx)).cuda()
    for flags in (0, _lib.SMLA_DKV_STORED_P, _lib.SMLA_DKV_ATOMIC):
        _, broken = guarded_step(q, kv, dout, idx, w.sm_scale, w.G, flags)
        assert not broken, f"flags {flags}: writes past the end of {broken}"


# ---------------------------------------------------------------------------
# Repeated-run stress
# ---------------------------------------------------------------------------

STRESS_ITERS = 50


def test_stress_repeated_backward():
    """50 calls of each backward form on one input, each checked before the
    next: the deterministic forms bit for bit against their first call, the
    atomic forms within fp32 rounding of the deterministic dkv; the first
    call of each form is also held to the oracle."""
    import bwd_sparse_mla_amd as smla
    w = synth.custom(S=512, H=16, K=512, S_kv=1100, seed=46, pad_frac=0.2, empty_frac=0.02,
                     dup_frac=0.01)
    print(f"[stress] S={w.S} H={w.H} K={w.K} S_kv={w.S_kv} x{STRESS_ITERS}", flush=True)
    q, kv, dout, idx = gpu_inputs(w)
    out, lse = smla.sparse_mla_fwd(q, kv, idx, w.sm_scale)
    ref32 = torch.empty(w.S_kv, 576, dtype=torch.float32, device="cuda")
    dq_ref, _ = smla.sparse_mla_bwd(q, kv, out, dout, idx, lse, w.sm_scale, dkv_f32=ref32)
    torch.cuda.synchronize()
    q64, kv64, do64 = oracle_inputs(w)
    s_dq, s_dkv = o_bwd(q64, kv64, do64, w.idx, w.sm_scale, out=bf16_to_np64(out),
                        lse=lse.cpu().numpy().astype(np.float64))
    assert rel_err(bf16_to_np64(dq_ref), s_dq) <= TOL
    assert rel_err(ref32.cpu().numpy().astype(np.float64), s_dkv) <= TOL
    scale = float(ref32.abs().max())
    # deterministic dkv of each backward form (the stored-P form rounds the
    # dq pass's P and dS to bf16, so its dkv differs from the recomputing
    # form's by that rounding): what the atomic form of each is held to
    det = {False: ref32, True: torch.empty_like(ref32)}
    smla.sparse_mla_bwd(q, kv, out, dout, idx, lse, w.sm_scale, dkv_f32=det[True], stored_p=True)
    for stored in (False, True):
        for atomic in (False, True):
            first = None
            d32 = torch.empty_like(ref32)
            for it in range(STRESS_ITERS):
                dq, dkv = smla.sparse_mla_bwd(q, kv, out, dout, idx, lse, w.sm_scale,
                                              dkv_f32=d32, atomic=atomic, stored_p=stored)
                torch.cuda.synchronize()
                tag = f"atomic={atomic} stored_p={stored} iteration {it}"
                assert torch.isfinite(d32).all() and torch.isfinite(dq.float()).all(), tag
                assert torch.equal(dq, dq_ref), tag
                if first is None:
                    first = (dq.clone(), d32.clone())
                    assert rel_err(bf16_to_np64(dq), s_dq) <= TOL, tag
                    assert rel_err(d32.cpu().numpy().astype(np.float64), s_dkv) <= TOL, tag
                if atomic:
                    err = float((d32 - det[stored]).abs().max())
                    assert err <= 1e-5 * scale, f"{tag}: |atomic - deterministic| {err:.3e}"
                else:
                    assert torch.equal(dq, first[0]) and torch.equal(d32, first[1]), tag
            print(f"[stress] atomic={atomic} stored_p={stored}: {STRESS_ITERS} calls ok", flush=True)


# ---------------------------------------------------------------------------
# Flat kv rows past 2^32 / 576 elements
# ---------------------------------------------------------------------------

def test_kv_rows_beyond_32_bit_element_offsets():
    """kv rows whose element offset row * 576 exceeds 2^32 (rows >= 7,456,541):
    a few tokens select rows at the top of a 7.6M-row kv (8.8 GB); out, lse,
    dq and dkv of those rows match the oracle on the selected rows."""
    import bwd_sparse_mla_amd as smla
    S_kv = 7_600_000
    S, H, K = 24, 8, 96
    rng = np.random.default_rng(47)
    top = np.arange(S_kv - 4000, S_kv)
    low = np.arange(0, 2000)
    cand = np.concatenate([low, top])
    idx = np.stack([rng.choice(cand, K, replace=False) for _ in range(S)]).astype(np.int32)
    idx[rng.random(idx.shape) < 0.2] = -1
    used = np.unique(idx[idx >= 0]).astype(np.int64)
    print(f"[bigkv] S_kv={S_kv} rows used={used.size} max row={used.max()}", flush=True)
    q_bits = synth.f32_to_bf16_bits(rng.standard_normal((S, H, 576)).astype(np.float32))
    do_bits = synth.f32_to_bf16_bits(rng.standard_normal((S, H, 512)).astype(np.float32))
    used_bits = synth.f32_to_bf16_bits(rng.standard_normal((used.size, 576)).astype(np.float32))
    kv = torch.zeros(S_kv, 576, dtype=torch.bfloat16, device="cuda")
    used_t = torch.from_numpy(used).cuda()
    kv.index_copy_(0, used_t, torch.from_numpy(used_bits.view(np.int16)).view(torch.bfloat16).cuda())
    q = torch.from_numpy(q_bits.view(np.int16)).view(torch.bfloat16).cuda()
    dout = torch.from_numpy(do_bits.view(np.int16)).view(torch.bfloat16).cuda()
    idx_t = torch.from_numpy(idx).cuda()
    scale = synth.SM_SCALE
    out, lse = smla.sparse_mla_fwd(q, kv, idx_t, scale)
    dq, dkv = smla.sparse_mla_bwd(q, kv, out, dout, idx_t, lse, scale, stored_p=True)
    torch.cuda.synchronize()
    sel = dkv.index_select(0, used_t)
    dkv_used = sel.float().cpu().numpy().astype(np.float64)
    # rows no slot selects are exactly zero: every nonzero element is on a used row
    nz_all = int(torch.count_nonzero(dkv.view(torch.int16)).item())
    nz_used = int(torch.count_nonzero(sel.view(torch.int16)).item())
    del kv, dkv, sel
    # oracle over the compacted kv (rows renumbered to 0..len(used)-1)
    remap = np.full(S_kv, -1, dtype=np.int64)
    remap[used] = np.arange(used.size)
    cidx = np.where(idx >= 0, remap[np.maximum(idx, 0)], -1)
    kv64 = synth.bf16_bits_to_f64(used_bits)
    q64 = synth.bf16_bits_to_f64(q_bits)
    do64 = synth.bf16_bits_to_f64(do_bits)
    from oracle import sparse_mla_fwd as o_fwd
    r_out, r_lse = o_fwd(q64, kv64, cidx, scale)
    g_out = bf16_to_np64(out)
    g_lse = lse.cpu().numpy().astype(np.float64)
    s_dq, s_dkv = o_bwd(q64, kv64, do64, cidx, scale, out=g_out, lse=g_lse)
    errs = {"out": rel_err(g_out, r_out), "lse": rel_err(g_lse, r_lse),
            "dq": rel_err(bf16_to_np64(dq), s_dq), "dkv": rel_err(dkv_used, s_dkv)}
    print(f"[bigkv] rel errors {errs}", flush=True)
    for k, v in errs.items():
        assert v <= TOL, f"{k} relative error {v:.3e}"
    assert nz_all == nz_used > 0, "dkv written on a row no slot selects"
