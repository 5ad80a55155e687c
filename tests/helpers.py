"""Shared test helpers: moving seeded workloads to the GPU, running the oracle
on the same inputs, and the error metrics."""
from __future__ import annotations

import numpy as np

from workloads import synth

TOL = 3e-3   # per-tensor relative error bound (fp32-reference agreement on the pages)


def rel_err(x, ref) -> float:
    """Norm-wise relative error ||x - ref||_2 / ||ref||_2 in fp64 (0 if both are 0)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def to_torch_bf16(bits, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def bf16_to_np64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def gpu_inputs(w: synth.Workload, device="cuda"):
    import torch
    q = to_torch_bf16(w.q, device)
    kv = to_torch_bf16(w.kv, device)
    dout = to_torch_bf16(w.dout, device)
    idx = torch.from_numpy(np.ascontiguousarray(w.idx)).to(device)
    return q, kv, dout, idx


def oracle_inputs(w: synth.Workload):
    return (synth.bf16_bits_to_f64(w.q), synth.bf16_bits_to_f64(w.kv),
            synth.bf16_bits_to_f64(w.dout))


def clean_idx(idx: np.ndarray, s_kv: int) -> np.ndarray:
    """Indices with every entry outside [0, s_kv) replaced by -1 (the padding
    reading of a contract violation)."""
    out = idx.copy()
    out[(out < 0) | (out >= s_kv)] = -1
    return out
