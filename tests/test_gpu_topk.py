"""GPU parity of the index-production top-k (through the C ABI) against the
oracle: bit-exact index rows on ranges of every kind (empty, shorter than K,
exactly K, just over K, far over K, past the row end), rows full of ties,
strided rows, rows too long to keep in LDS, and the indices feeding the
attention; at full size, sampled rows of a single 8192-token sequence with
K = 2048 in the launch configuration the benchmark times."""
import numpy as np
import pytest

from oracle import causal_ranges, sparse_mla_fwd as o_fwd, topk_indices as o_topk
from tests.helpers import TOL, bf16_to_np64, gpu_inputs, oracle_inputs, rel_err
from workloads import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bwd_sparse_mla_amd
    bwd_sparse_mla_amd.load_library()


def _gpu_topk(logits_np, ks, ke, K, ld=None):
    import bwd_sparse_mla_amd as smla
    S, S_kv = logits_np.shape
    if ld is None:
        lg = torch.from_numpy(np.ascontiguousarray(logits_np)).cuda()
    else:   # rows ld apart, columns past S_kv hold junk the kernel must not read
        big = np.full((S, ld), np.nan, dtype=np.float32)
        big[:, :S_kv] = logits_np
        lg = torch.from_numpy(big).cuda()[:, :S_kv]
    out = smla.topk_indices(lg, torch.from_numpy(ks).cuda(), torch.from_numpy(ke).cuda(), K)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_ranges_of_every_kind(seed):
    rng = np.random.default_rng(seed)
    S, S_kv, K = 64, 700, 96
    logits = rng.standard_normal((S, S_kv)).astype(np.float32)
    lens = np.array([0, 1, 5, 95, 96, 97, 98, 191, 192, 500, 700, 690] * 6)[:S - 4]
    ks = rng.integers(0, S_kv, S).astype(np.int32)
    ks[:len(lens)] = np.minimum(ks[:len(lens)], S_kv - lens)
    ke = ks.copy()
    ke[:len(lens)] = ks[:len(lens)] + lens
    ke[-4:] = [ks[-4] - 3, S_kv + 50, ks[-2], S_kv]    # empty (ke < ks), past the end, empty, to the end
    print(f"[topk] ranges seed={seed} S={S} S_kv={S_kv} K={K}", flush=True)
    got = _gpu_topk(logits, ks, ke, K)
    np.testing.assert_array_equal(got, o_topk(logits, ks, ke, K))


def test_ties_and_strided_rows():
    rng = np.random.default_rng(5)
    S, S_kv, K = 48, 520, 64
    logits = rng.integers(-3, 4, (S, S_kv)).astype(np.float32)   # heavy ties
    logits[0] = 1.0                                             # one value everywhere
    logits[1, ::2] = -0.0                                       # signed zeros tie with +0
    ks = np.zeros(S, dtype=np.int32)
    ke = np.full(S, S_kv, dtype=np.int32)
    ke[5:] = rng.integers(60, S_kv, S - 5)
    print(f"[topk] ties S={S} S_kv={S_kv} K={K} ld=600", flush=True)
    got = _gpu_topk(logits, ks, ke, K, ld=600)
    np.testing.assert_array_equal(got, o_topk(logits, ks, ke, K))


def test_rows_longer_than_the_lds_cache():
    rng = np.random.default_rng(6)
    S, S_kv, K = 4, 40000, 2048
    logits = rng.standard_normal((S, S_kv)).astype(np.float32)
    ks = np.array([0, 100, 7000, 0], dtype=np.int32)
    ke = np.array([40000, 39000, 40000, 32768], dtype=np.int32)
    print(f"[topk] long rows S_kv={S_kv} K={K}", flush=True)
    got = _gpu_topk(logits, ks, ke, K)
    np.testing.assert_array_equal(got, o_topk(logits, ks, ke, K))


def test_small_k_every_alignment():
    """K = 1, 2, 3 over short rows starting at every offset mod 4 (the kernel
    reads each row's unaligned head one by one, the body as 16-byte loads)."""
    rng = np.random.default_rng(9)
    S, S_kv = 96, 37
    logits = rng.standard_normal((S, S_kv)).astype(np.float32)
    logits[::7] = np.round(logits[::7])                 # some rows with ties
    ks = (np.arange(S) % 8).astype(np.int32)
    ke = np.minimum(S_kv, ks + 2 + (np.arange(S) // 8) % 9).astype(np.int32)
    for K in (1, 2, 3):
        print(f"[topk] small K={K} S={S} S_kv={S_kv}", flush=True)
        got = _gpu_topk(logits, ks, ke, K)
        np.testing.assert_array_equal(got, o_topk(logits, ks, ke, K))


def test_rows_between_the_two_cache_sizes():
    """S_kv just past 8192: rows of 8193..9000 keys use the larger LDS cache."""
    rng = np.random.default_rng(10)
    S, S_kv, K = 6, 9000, 2048
    logits = rng.standard_normal((S, S_kv)).astype(np.float32)
    ks = np.array([0, 1, 2, 3, 0, 500], dtype=np.int32)
    ke = np.array([9000, 8194, 9000, 8999, 8192, 9000], dtype=np.int32)
    print(f"[topk] medium rows S_kv={S_kv} K={K}", flush=True)
    got = _gpu_topk(logits, ks, ke, K)
    np.testing.assert_array_equal(got, o_topk(logits, ks, ke, K))


def test_indices_feed_the_attention():
    """topk -> sparse_mla_fwd equals the oracle's forward on the oracle's
    selection (packed causal sequences, rows shorter and longer than K)."""
    import bwd_sparse_mla_amd as smla
    rng = np.random.default_rng(7)
    seqlens = [90, 150, 60]
    ks, ke = causal_ranges(seqlens)
    S = len(ks)
    K = 64
    logits = rng.standard_normal((S, S)).astype(np.float32)
    idx_ref = o_topk(logits, ks, ke, K)
    idx_gpu = _gpu_topk(logits, ks, ke, K)
    np.testing.assert_array_equal(idx_gpu, idx_ref)
    w = synth.custom(S=S, H=16, K=K, S_kv=S, seed=8)
    w.idx = idx_ref
    q, kv, dout, idx = gpu_inputs(w)
    out, lse = smla.sparse_mla_fwd(q, kv, torch.from_numpy(idx_gpu).cuda(), w.sm_scale)
    torch.cuda.synchronize()
    q64, kv64, _ = oracle_inputs(w)
    r_out, r_lse = o_fwd(q64, kv64, idx_ref, w.sm_scale)
    assert rel_err(bf16_to_np64(out), r_out) <= TOL
    assert rel_err(lse.cpu().numpy().astype(np.float64), r_lse) <= TOL


def test_full_size_single_sequence_sampled():
    """S = 8192 causal rows of one sequence, K = 2048: every row checked for
    shape and validity, sampled rows bit-exact against the oracle."""
    import bwd_sparse_mla_amd as smla
    S, K = 8192, 2048
    gen = torch.Generator(device="cuda").manual_seed(9)
    lg = torch.randn(S, S, device="cuda", generator=gen, dtype=torch.float32)
    ks_np, ke_np = causal_ranges([S])
    ks, ke = torch.from_numpy(ks_np).cuda(), torch.from_numpy(ke_np).cuda()
    print(f"[topk] full size S={S} K={K}", flush=True)
    out = smla.topk_indices(lg, ks, ke, K)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    n = np.minimum(ke_np - ks_np, K)
    cols = np.arange(K)[None, :]
    valid = cols < n[:, None]
    assert np.all(o[~valid] == -1)
    assert np.all((o[valid] >= 0) & (o[valid] < np.repeat(ke_np[:, None], K, 1)[valid]))
    assert np.all(np.diff(o, axis=1)[valid[:, 1:]] > 0), "chosen positions not ascending"
    rows = np.unique(np.concatenate([[0, 1, 2047, 2048, 2049, 4095, S - 1],
                                     np.random.default_rng(10).choice(S, 12, replace=False)]))
    lg_rows = lg[torch.from_numpy(rows).cuda()].cpu().numpy()
    ref = o_topk(lg_rows, ks_np[rows], ke_np[rows], K)
    np.testing.assert_array_equal(o[rows], ref)
