"""GPU parity of the nonfinite diagnostics (through the C ABI) against the
oracle: exact counts and bit-exact replacement on bf16 and fp32 buffers with
planted NaN / Inf of every kind, at sizes with ragged tails (0, 1, 7, 8, 9,
~1e6 + 3, 2^22 + 5 elements), with and without a reference; the count adds
into the caller's counter; and the checked backward on the packed ragged
workload (finite, so nothing to replace) and with NaN planted in its dq."""
import numpy as np
import pytest

from oracle import count_nonfinite as o_count, replace_nonfinite as o_replace
from tests.helpers import gpu_inputs
from workloads import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TORCH_T = {"bf16": torch.int16, "f32": torch.int32}
VIEW_T = {"bf16": torch.bfloat16, "f32": torch.float32}
NP_T = {"bf16": np.int16, "f32": np.int32}


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bwd_sparse_mla_amd
    bwd_sparse_mla_amd.load_library()


def to_gpu(bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(NP_T[dtype])).cuda()
    return t.view(VIEW_T[dtype])


def to_bits(t, dtype):
    return t.view(TORCH_T[dtype]).cpu().numpy().view(np.uint16 if dtype == "bf16" else np.uint32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 1000003, (1 << 22) + 5])
def test_count_and_replace(dtype, n):
    import bwd_sparse_mla_amd as smla
    bits, ref = synth.planted_nonfinite(n, dtype, frac=0.02 if n > 100 else 0.4, seed=n % 97)
    print(f"[diag] dtype={dtype} n={n}", flush=True)
    x = to_gpu(bits, dtype)
    r = to_gpu(ref, dtype)
    assert smla.count_nonfinite(x) == o_count(bits, dtype)
    want, nrep = o_replace(bits, ref, dtype)
    got = smla.replace_nonfinite_(x, r)
    assert got == nrep
    assert np.array_equal(to_bits(x, dtype), want)
    assert smla.count_nonfinite(x) == 0
    z = to_gpu(bits, dtype)
    want0, n0 = o_replace(bits, None, dtype)
    assert smla.replace_nonfinite_(z) == n0
    assert np.array_equal(to_bits(z, dtype), want0)


def test_counter_accumulates_and_offsets():
    """The count is added into the caller's counter; sub-buffers starting at
    16-byte offsets are counted on their own."""
    import bwd_sparse_mla_amd as smla
    bits, _ = synth.planted_nonfinite(50000, "f32", frac=0.01, seed=11)
    x = to_gpu(bits, "f32")
    c = torch.full((1,), 5, dtype=torch.int64, device="cuda")
    smla.count_nonfinite(x, c)
    smla.count_nonfinite(x[4:], c)
    torch.cuda.synchronize()
    assert int(c.item()) == 5 + o_count(bits, "f32") + o_count(bits[4:], "f32")


def test_checked_backward():
    import bwd_sparse_mla_amd as smla
    w = synth.packed_ragged()
    print(f"[diag] checked backward on {w.name}", flush=True)
    q, kv, dout, idx = gpu_inputs(w)
    out, lse = smla.sparse_mla_fwd(q, kv, idx, w.sm_scale)
    dq, dkv, info = smla.sparse_mla_bwd_checked(q, kv, out, dout, idx, lse, w.sm_scale)
    assert info == {"dq": 0, "dkv": 0, "replaced": 0}
    # NaN planted into a copy of dq is restored from the clean result, bit for bit
    bad = dq.clone()
    flat = bad.view(-1)
    pos = torch.arange(0, flat.numel(), 9973, device="cuda")
    flat[pos] = float("nan")
    flat[pos[::2] + 1] = float("inf")
    n_bad = int(pos.numel() + pos[::2].numel())
    assert smla.count_nonfinite(bad) == n_bad
    assert smla.replace_nonfinite_(bad, dq) == n_bad
    assert torch.equal(bad.view(torch.int16), dq.view(torch.int16))
    # with a reference callable, the checked call takes it only where needed
    calls = []

    def reference(*args):
        calls.append(1)
        return dq, dkv

    dq2, dkv2, info2 = smla.sparse_mla_bwd_checked(q, kv, out, dout, idx, lse, w.sm_scale,
                                                   reference=reference)
    assert info2["replaced"] == 0 and not calls
    assert torch.equal(dq2.view(torch.int16), dq.view(torch.int16))
