"""GPU parity of the fp8 kv forward (smla_fwd_fp8: 656-byte records of e4m3
latent codes, per-128-column fp32 scales and bf16 rope):

  * bit for bit equal to the bf16 forward over the decoded rows when every
    decoded value is exact in bf16 (power-of-two scales), on records that
    walk through every non-NaN e4m3 code: the decode of every code, the
    record layout and the tile placement -- with the general conversion and
    with the one-instruction conversion for power-of-two scales;
  * against the oracle (decode to bf16 rows, then the fp64 forward) with
    fp32 scales (amax / 448), padding, empty rows and out-of-range indices,
    and bit for bit against the bf16 forward over the oracle's decoded rows;
  * with several kv groups and 128 heads per group, against the grouped
    oracle; the plan built once gives the one-shot result bit for bit;
  * at the full size of the packed ragged batch in the bench's launch
    configuration: bit for bit the bf16 forward over the decoded rows, and
    sampled tokens against the oracle.
"""
import numpy as np
import pytest

from oracle import EMPTY_ROW_LSE, decode_kv_records, kv_rows_bf16, sparse_mla_fwd_fp8
from tests.helpers import TOL, bf16_to_np64, rel_err, to_torch_bf16
from workloads import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bwd_sparse_mla_amd
    bwd_sparse_mla_amd.load_library()


def _clean(idx, s_kv):
    return np.where((idx >= 0) & (idx < s_kv), idx, -1).astype(np.int32)


def _all_code_records(s_kv, seed):
    rng = np.random.default_rng(seed)
    j = np.arange(s_kv)[:, None]
    c = np.arange(512)[None, :]
    codes = ((j * 37 + c * 5) % 256).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x00                 # no NaN codes
    rec = np.zeros((s_kv, 656), dtype=np.uint8)
    rec[:, :512] = codes
    scales = np.exp2(rng.integers(-6, 4, size=(s_kv, 4))).astype("<f4")
    rec[:, 512:528] = scales.view(np.uint8).reshape(s_kv, 16)
    rope = synth.f32_to_bf16_bits(rng.standard_normal((s_kv, 64)).astype(np.float32))
    rec[:, 528:] = rope.astype("<u2").view(np.uint8).reshape(s_kv, 128)
    return rec


def test_fp8_forward_is_the_bf16_forward_on_exact_decoded_rows():
    import bwd_sparse_mla_amd as smla
    w = synth.custom(S=40, H=16, K=96, S_kv=300, seed=51, pad_frac=0.2, empty_frac=0.1)
    rec = _all_code_records(w.S_kv, 52)
    kv64 = decode_kv_records(rec)
    kv_bits = synth.f32_to_bf16_bits(kv64.astype(np.float32))
    assert np.array_equal(synth.bf16_bits_to_f64(kv_bits), kv64)      # exact in bf16
    print(f"[fp8] all codes S={w.S} H={w.H} K={w.K} S_kv={w.S_kv}", flush=True)
    q = to_torch_bf16(w.q)
    idx = torch.from_numpy(w.idx).cuda()
    k8 = torch.from_numpy(rec).cuda()
    out8, lse8 = smla.sparse_mla_fwd_fp8(q, k8, idx, w.sm_scale)
    out2, lse2 = smla.sparse_mla_fwd_fp8(q, k8, idx, w.sm_scale, pow2_scales=True)
    out, lse = smla.sparse_mla_fwd(q, to_torch_bf16(kv_bits), idx, w.sm_scale)
    torch.cuda.synchronize()
    for o, l in ((out8, lse8), (out2, lse2)):   # fp32-scale and power-of-two-scale conversions
        assert torch.equal(o.view(torch.int16), out.view(torch.int16))
        assert torch.equal(l.view(torch.int32), lse.view(torch.int32))


CASES = {
    "h8_oob": dict(S=70, H=8, K=200, S_kv=600, seed=53, pad_frac=0.3, empty_frac=0.05,
                   oob_frac=0.03),
    "h64_dups": dict(S=20, H=64, K=150, S_kv=400, seed=54, pad_frac=0.2, dup_frac=0.1),
    "h128": dict(S=11, H=128, K=300, S_kv=900, seed=55, pad_frac=0.1, empty_frac=0.1),
}


@pytest.mark.parametrize("case", list(CASES))
def test_fp8_forward_against_the_oracle(case):
    import bwd_sparse_mla_amd as smla
    w = synth.custom(**CASES[case])
    rec = synth.quantize_kv_fp8(w.kv, pow2_scales=False)
    print(f"[fp8] {case} S={w.S} H={w.H} K={w.K} S_kv={w.S_kv}", flush=True)
    q, idx = to_torch_bf16(w.q), torch.from_numpy(w.idx).cuda()
    out, lse = smla.sparse_mla_fwd_fp8(q, torch.from_numpy(rec).cuda(), idx, w.sm_scale)
    kv_bits = synth.f32_to_bf16_bits(kv_rows_bf16(rec).astype(np.float32))   # exact
    out_b, lse_b = smla.sparse_mla_fwd(q, to_torch_bf16(kv_bits), idx, w.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_b.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse_b.view(torch.int32))
    oidx = _clean(w.idx, w.S_kv)
    r_out, r_lse = sparse_mla_fwd_fp8(synth.bf16_bits_to_f64(w.q), rec, oidx, w.sm_scale)
    g_out, g_lse = bf16_to_np64(out), lse.cpu().numpy().astype(np.float64)
    e_out, e_lse = rel_err(g_out, r_out), rel_err(g_lse, r_lse)
    print(f"[fp8] {case} rel errors out {e_out:.3e} lse {e_lse:.3e}", flush=True)
    assert e_out <= TOL and e_lse <= TOL
    empty = ~(oidx >= 0).any(axis=1)
    if empty.any():
        assert np.all(g_out[empty] == 0.0)
        np.testing.assert_allclose(g_lse[empty], EMPTY_ROW_LSE, rtol=1e-6)


@pytest.mark.parametrize("H", [256, 16])   # 128 heads per group; 8 (group-major staging)
def test_fp8_forward_with_kv_groups_and_the_plan_built_once(H):
    import bwd_sparse_mla_amd as smla
    w = synth.custom_grouped(S=9 if H == 256 else 40, H=H, G=2, K=100, S_kv=200, seed=56,
                             pad_frac=0.25, empty_frac=0.1)
    rec = synth.quantize_kv_fp8(w.kv, pow2_scales=False)            # [S_kv, G, 656]
    print(f"[fp8] kv groups S={w.S} H={w.H} G={w.G} K={w.K}", flush=True)
    q = to_torch_bf16(w.q)
    k8 = torch.from_numpy(rec).cuda()
    idx = torch.from_numpy(np.ascontiguousarray(w.idx)).cuda()
    out, lse = smla.sparse_mla_fwd_fp8(q, k8, idx, w.sm_scale)
    run = smla.SparseMLARunner(w.S, w.S_kv, w.H, w.K, q.device, kv_groups=w.G)
    run.plan(idx)
    run.fwd_fp8(q, k8, idx, w.sm_scale, planned=True)
    torch.cuda.synchronize()
    assert torch.equal(run.out.view(torch.int16), out.view(torch.int16))
    assert torch.equal(run.lse.view(torch.int32), lse.view(torch.int32))
    oidx = _clean(w.idx, w.S_kv)
    r_out, r_lse = sparse_mla_fwd_fp8(synth.bf16_bits_to_f64(w.q), rec, oidx, w.sm_scale)
    e_out = rel_err(bf16_to_np64(out), r_out)
    e_lse = rel_err(lse.cpu().numpy().astype(np.float64), r_lse)
    print(f"[fp8] kv groups rel errors out {e_out:.3e} lse {e_lse:.3e}", flush=True)
    assert e_out <= TOL and e_lse <= TOL


def test_fp8_forward_full_size_in_the_bench_configuration():
    # the packed ragged batch (S = 4096, H = 8, topk = 2048) through the
    # runner with the plan built once, as the bench times it: bit for bit the
    # bf16 forward over the oracle's decoded rows, and sampled tokens against
    # the oracle
    import bwd_sparse_mla_amd as smla
    from oracle import sparse_mla_fwd
    w = synth.WORKLOADS["packed_ragged"]()
    print(f"[fp8] full size {w.name}", flush=True)
    rec = synth.quantize_kv_fp8(w.kv, pow2_scales=False)
    kv64 = kv_rows_bf16(rec)
    kv_bits = synth.f32_to_bf16_bits(kv64.astype(np.float32))
    q, idx = to_torch_bf16(w.q), torch.from_numpy(np.ascontiguousarray(w.idx)).cuda()
    run = smla.SparseMLARunner(w.S, w.S_kv, w.H, w.K, q.device)
    run.plan(idx)
    out8, lse8 = (t.clone() for t in run.fwd_fp8(q, torch.from_numpy(rec).cuda(), idx,
                                                 w.sm_scale, planned=True))
    out, lse = run.fwd(q, to_torch_bf16(kv_bits), idx, w.sm_scale, planned=True)
    torch.cuda.synchronize()
    assert torch.equal(out8.view(torch.int16), out.view(torch.int16))
    assert torch.equal(lse8.view(torch.int32), lse.view(torch.int32))
    rng = np.random.default_rng(7)
    ends = np.cumsum(w.seqlens) - 1
    toks = np.unique(np.concatenate([ends, rng.choice(w.S, 12, replace=False)]))
    r_out, r_lse = sparse_mla_fwd(synth.bf16_bits_to_f64(w.q[toks]), kv64, w.idx[toks],
                                  w.sm_scale)
    sel = torch.as_tensor(toks, device="cuda")
    e_out = rel_err(bf16_to_np64(out8.index_select(0, sel)), r_out)
    e_lse = rel_err(lse8.index_select(0, sel).cpu().numpy().astype(np.float64), r_lse)
    print(f"[fp8] full size sampled rel errors out {e_out:.3e} lse {e_lse:.3e}", flush=True)
    assert e_out <= TOL and e_lse <= TOL


def test_fp8_power_of_two_scales_full_size():
    # power-of-two scales at the packed ragged batch's full size: the
    # one-instruction conversion gives the general conversion's result and
    # the bf16 forward's over the decoded rows, bit for bit
    import bwd_sparse_mla_amd as smla
    w = synth.WORKLOADS["packed_ragged"]()
    print(f"[fp8] power-of-two scales, full size {w.name}", flush=True)
    rec = synth.quantize_kv_fp8(w.kv, pow2_scales=True)
    kv_bits = synth.f32_to_bf16_bits(kv_rows_bf16(rec).astype(np.float32))
    q, idx = to_torch_bf16(w.q), torch.from_numpy(np.ascontiguousarray(w.idx)).cuda()
    k8 = torch.from_numpy(rec).cuda()
    run = smla.SparseMLARunner(w.S, w.S_kv, w.H, w.K, q.device)
    run.plan(idx)
    o2, l2 = (t.clone() for t in run.fwd_fp8(q, k8, idx, w.sm_scale, planned=True,
                                             pow2_scales=True))
    o1, l1 = (t.clone() for t in run.fwd_fp8(q, k8, idx, w.sm_scale, planned=True))
    ob, lb = run.fwd(q, to_torch_bf16(kv_bits), idx, w.sm_scale, planned=True)
    torch.cuda.synchronize()
    for o, l in ((o2, l2), (o1, l1)):
        assert torch.equal(o.view(torch.int16), ob.view(torch.int16))
        assert torch.equal(l.view(torch.int32), lb.view(torch.int32))


def test_runner_rejects_wrong_inputs_before_launching():
    import bwd_sparse_mla_amd as smla
    run = smla.SparseMLARunner(8, 64, 8, 16, "cuda")
    q = torch.zeros(8, 8, 576, dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros(8, 16, dtype=torch.int32, device="cuda")
    kv = torch.zeros(64, 576, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        run.fwd(q[:, :4].contiguous(), kv, idx, 0.1)                       # wrong heads
    with pytest.raises(ValueError):
        run.fwd(q, kv[:32].contiguous(), idx, 0.1)                         # wrong s_kv
    with pytest.raises(ValueError):
        run.plan(idx.to(torch.int64))                                      # wrong dtype
    with pytest.raises(ValueError):
        run.fwd_fp8(q, torch.zeros(63, 656, dtype=torch.uint8, device="cuda"), idx, 0.1)
    with pytest.raises(ValueError):
        run.bwd(q, kv, torch.zeros(8, 8, 512, dtype=torch.bfloat16, device="cuda").transpose(0, 1), idx,
                0.1)
