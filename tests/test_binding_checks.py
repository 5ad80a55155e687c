"""The Python binding rejects caller-supplied buffers the kernels would write
outside of (wrong device, dtype, size or layout) before anything is launched.

Runs without a GPU: the binding's device type is pointed at "cpu" and the
library at a stand-in that answers the workspace queries and fails the test
on any launching call.
"""
import pytest
import torch

from bwd_sparse_mla_amd import ops

S, H, K, S_KV = 6, 8, 4, 10


class NoLaunchLib:
    """Workspace queries answer; every other entry point is a launch."""

    def smla_fwd_workspace_size_g(self, *args):
        return 4096

    def smla_bwd_workspace_size_g(self, *args):
        return 4096

    def __getattr__(self, name):
        def launch(*args):
            raise AssertionError(f"{name} was called although an argument was invalid")
        return launch


@pytest.fixture
def cpu_binding(monkeypatch):
    monkeypatch.setattr(ops, "_DEVICE_TYPE", "cpu")
    monkeypatch.setattr(ops._lib, "load", lambda: NoLaunchLib())
    monkeypatch.setattr(ops, "_stream", lambda device: None)


def inputs():
    q = torch.zeros(S, H, 576, dtype=torch.bfloat16)
    kv = torch.zeros(S_KV, 576, dtype=torch.bfloat16)
    idx = torch.full((S, K), -1, dtype=torch.int32)
    out = torch.zeros(S, H, 512, dtype=torch.bfloat16)
    lse = torch.zeros(S, H, dtype=torch.float32)
    return q, kv, idx, out, lse


BAD_OUT = {
    "short": torch.zeros(S, H, 511, dtype=torch.bfloat16),
    "fp32": torch.zeros(S, H, 512, dtype=torch.float32),
    "strided": torch.zeros(S, H, 1024, dtype=torch.bfloat16)[..., ::2],
    "meta": torch.empty(S, H, 512, dtype=torch.bfloat16, device="meta"),
}
BAD_LSE = {
    "short": torch.zeros(S, H - 1, dtype=torch.float32),
    "bf16": torch.zeros(S, H, dtype=torch.bfloat16),
    "strided": torch.zeros(S, 2 * H, dtype=torch.float32)[:, ::2],
    "meta": torch.empty(S, H, dtype=torch.float32, device="meta"),
}


@pytest.mark.parametrize("kind", sorted(BAD_OUT))
def test_fwd_rejects_bad_out(cpu_binding, kind):
    q, kv, idx, _, _ = inputs()
    with pytest.raises(ValueError):
        ops.sparse_mla_fwd(q, kv, idx, 0.1, out=BAD_OUT[kind])


@pytest.mark.parametrize("kind", sorted(BAD_LSE))
def test_fwd_rejects_bad_lse(cpu_binding, kind):
    q, kv, idx, _, _ = inputs()
    with pytest.raises(ValueError):
        ops.sparse_mla_fwd(q, kv, idx, 0.1, lse=BAD_LSE[kind])


@pytest.mark.parametrize("kind", sorted(BAD_OUT))
def test_fp8_fwd_rejects_bad_out(cpu_binding, kind):
    q, _, idx, _, _ = inputs()
    kv8 = torch.zeros(S_KV, 656, dtype=torch.uint8)
    with pytest.raises(ValueError):
        ops.sparse_mla_fwd_fp8(q, kv8, idx, 0.1, out=BAD_OUT[kind])


BAD_DKV32 = {
    "short": torch.zeros(S_KV * 576 - 4, dtype=torch.float32),
    "bf16": torch.zeros(S_KV, 576, dtype=torch.bfloat16),
    "strided": torch.zeros(S_KV, 1152, dtype=torch.float32)[:, ::2],
    "meta": torch.empty(S_KV, 576, dtype=torch.float32, device="meta"),
}


@pytest.mark.parametrize("kind", sorted(BAD_DKV32))
def test_bwd_rejects_bad_dkv_f32(cpu_binding, kind):
    q, kv, idx, out, lse = inputs()
    with pytest.raises(ValueError):
        ops.sparse_mla_bwd(q, kv, out, out.clone(), idx, lse, 0.1, dkv_f32=BAD_DKV32[kind])


@pytest.mark.parametrize("which", ["out", "dout", "lse"])
def test_bwd_rejects_wrong_sized_inputs(cpu_binding, which):
    q, kv, idx, out, lse = inputs()
    args = {"out": out, "dout": out.clone(), "lse": lse}
    args[which] = args[which][:-1]
    with pytest.raises(ValueError):
        ops.sparse_mla_bwd(q, kv, args["out"], args["dout"], idx, args["lse"], 0.1)


def test_inputs_on_another_device_are_rejected(cpu_binding):
    q, kv, idx, out, lse = inputs()
    with pytest.raises(ValueError):
        ops.sparse_mla_fwd(q, kv.to("meta"), idx, 0.1)
    with pytest.raises(ValueError):
        ops.sparse_mla_bwd(q, kv, out, out.clone(), idx, lse.to("meta"), 0.1)


def test_topk_rejects_bad_out(cpu_binding):
    logits = torch.zeros(S, S_KV, dtype=torch.float32)
    ks = torch.zeros(S, dtype=torch.int32)
    ke = torch.full((S,), S_KV, dtype=torch.int32)
    with pytest.raises(ValueError):
        ops.topk_indices(logits, ks, ke, K, out=torch.zeros(S, K - 1, dtype=torch.int32))
    with pytest.raises(ValueError):
        ops.topk_indices(logits, ks, ke, K, out=torch.zeros(S, K, dtype=torch.int64))


def test_valid_buffers_reach_the_launch(cpu_binding):
    """The stand-in library's launch is reached with valid buffers, so the
    rejections above come from the binding's checks."""
    q, kv, idx, out, lse = inputs()
    with pytest.raises(AssertionError, match="smla_fwd_g"):
        ops.sparse_mla_fwd(q, kv, idx, 0.1, out=out, lse=lse)
    with pytest.raises(AssertionError, match="smla_bwd_g"):
        ops.sparse_mla_bwd(q, kv, out, out.clone(), idx, lse, 0.1,
                           dkv_f32=torch.zeros(S_KV, 576, dtype=torch.float32))
