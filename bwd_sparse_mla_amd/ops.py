"""Python binding of libsmla: argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI
(include/smla.h).  PyTorch provides device memory and the current stream.

Accepted layouts (packed "thd" tokens, one KV group):
  q        [S, H, 576]  or [1, S, H, 576]                bf16
  kv       [S_kv, 576], [S_kv, 1, 576] or [1, S_kv, 1, 576]  bf16
  indices  [S, K], [S, 1, K] or [1, S, 1, K]            int32 or int64 (-1 = padding)
  dout     like out: q's leading dims + (512,)           bf16
Outputs keep the caller's leading dims: out [..., 512], lse [..., H] fp32,
dq like q, dkv like kv.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib

D_V = 512
D_K = 576


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _flat_q(q: torch.Tensor) -> torch.Tensor:
    if q.dim() == 4:
        if q.shape[0] != 1:
            raise ValueError("q with a batch dimension must have batch 1 (packed layout)")
        q = q[0]
    if q.dim() != 3 or q.shape[-1] != D_K:
        raise ValueError(f"q must be [S, H, {D_K}], got {tuple(q.shape)}")
    return q


def _grouped_kv(kv: torch.Tensor) -> tuple[torch.Tensor, int]:
    """kv as [S_kv, G, 576] (G = 1 for [S_kv, 576]); returns (kv, G)."""
    if kv.dim() == 4:
        if kv.shape[0] != 1:
            raise ValueError("kv with a batch dimension must have batch 1")
        kv = kv[0]
    if kv.dim() == 2:
        kv = kv.unsqueeze(1)
    if kv.dim() != 3 or kv.shape[-1] != D_K:
        raise ValueError(f"kv must be [S_kv, {D_K}] or [S_kv, G, {D_K}], got {tuple(kv.shape)}")
    return kv, kv.shape[1]


def _grouped_idx(idx: torch.Tensor, groups: int) -> torch.Tensor:
    """indices as [S, G, K] ([S, K] when G = 1)."""
    if idx.dim() == 4:
        if idx.shape[0] != 1:
            raise ValueError("indices with a batch dimension must have batch 1")
        idx = idx[0]
    if idx.dim() == 2 and groups == 1:
        idx = idx.unsqueeze(1)
    if idx.dim() != 3 or idx.shape[1] != groups:
        raise ValueError(f"indices must be [S, {groups}, K] for {groups} KV group(s), "
                         f"got {tuple(idx.shape)}")
    return idx


# Device type the kernels run on (a test on a machine without a GPU may point
# it at "cpu" together with a stand-in library to reach the checks below).
_DEVICE_TYPE = "cuda"


def _on_device(t: torch.Tensor, device: torch.device | None) -> bool:
    return t.device.type == _DEVICE_TYPE and (device is None or t.device == device)


def _prep(t: torch.Tensor, dtype: torch.dtype, name: str,
          device: torch.device | None = None) -> torch.Tensor:
    if not _on_device(t, device):
        raise ValueError(f"{name} must be a GPU tensor" + (f" on {device}" if device else ""))
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.contiguous()


def _dest(t: torch.Tensor, dtype: torch.dtype, numel: int, device: torch.device,
          name: str) -> torch.Tensor:
    """A buffer the caller hands in for the kernels to write: it must be
    exactly what they write (device, dtype, element count, contiguous), or
    the kernels would write outside it; checked before any launch."""
    if not isinstance(t, torch.Tensor) or not _on_device(t, device):
        raise ValueError(f"{name} must be a GPU tensor on {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()}")
    return t


def _workspace(nbytes: int, device) -> tuple[torch.Tensor, int]:
    """A device buffer of nbytes with a 256-byte aligned start; returns
    (owner tensor, aligned address)."""
    buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    addr = buf.data_ptr()
    return buf, (addr + 255) & ~255


def fwd_workspace_bytes(s_q: int, s_kv: int, heads: int, topk: int, kv_groups: int = 1) -> int:
    n = _lib.load().smla_fwd_workspace_size_g(s_q, s_kv, heads, kv_groups, topk)
    if n == 0:
        raise ValueError("unsupported shape for smla_fwd")
    return n


def bwd_workspace_bytes(s_q: int, s_kv: int, heads: int, topk: int, flags: int = 0,
                        kv_groups: int = 1) -> int:
    n = _lib.load().smla_bwd_workspace_size_g(s_q, s_kv, heads, kv_groups, topk, flags)
    if n == 0:
        raise ValueError("unsupported shape for smla_bwd")
    return n


def sparse_mla_fwd(q: torch.Tensor, kv: torch.Tensor, indices: torch.Tensor, sm_scale: float,
                   out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """Forward: returns (out [..., H, 512] bf16, lse [..., H] fp32, natural log).

    kv is [S_kv, 576] or [S_kv, G, 576] with G KV groups; indices are [S, K]
    or [S, G, K]; head h attends over kv group h // (H // G)."""
    lib = _lib.load()
    lead = q.shape[:-1]
    q3 = _prep(_flat_q(q), torch.bfloat16, "q")
    kv3, G = _grouped_kv(kv)
    kv3 = _prep(kv3, torch.bfloat16, "kv", q3.device)
    ix = _grouped_idx(indices, G)
    if ix.dtype != torch.int32:
        ix = ix.to(torch.int32)
    ix = _prep(ix, torch.int32, "indices", q3.device)
    S, H, _ = q3.shape
    if ix.shape[0] != S:
        raise ValueError("indices must have one row per query token")
    K = ix.shape[2]
    S_kv = kv3.shape[0]
    dev = q3.device
    if out is None:
        out = torch.empty(*lead[:-1], H, D_V, dtype=torch.bfloat16, device=dev)
    else:
        _dest(out, torch.bfloat16, S * H * D_V, dev, "out")
    if lse is None:
        lse = torch.empty(*lead[:-1], H, dtype=torch.float32, device=dev)
    else:
        _dest(lse, torch.float32, S * H, dev, "lse")
    ws, ws_addr = _workspace(fwd_workspace_bytes(S, S_kv, H, K, G), dev)
    _lib.check(lib.smla_fwd_g(_ptr(q3), _ptr(kv3), _ptr(ix), S, S_kv, H, G, K, float(sm_scale),
                              _ptr(out), _ptr(lse), 0, ctypes.c_void_p(ws_addr),
                              ws.numel() - (ws_addr - ws.data_ptr()), _stream(dev)))
    return out, lse


FP8_REC_BYTES = 656


def sparse_mla_fwd_fp8(q: torch.Tensor, kv_fp8: torch.Tensor, indices: torch.Tensor,
                       sm_scale: float, out: torch.Tensor | None = None,
                       lse: torch.Tensor | None = None, pow2_scales: bool = False):
    """Forward over fp8 kv records: kv_fp8 is uint8 [S_kv, 656] (or
    [S_kv, G, 656] with indices [S, G, K]), each row 512 e4m3 latent values,
    four fp32 scales (one per 128 columns) and the 64 bf16 rope values.
    pow2_scales=True promises that every scale is a power of two (faster
    conversion; other scales then give wrong values).  Returns (out, lse) as
    sparse_mla_fwd does."""
    lib = _lib.load()
    lead = q.shape[:-1]
    q3 = _prep(_flat_q(q), torch.bfloat16, "q")
    k8 = kv_fp8[0] if kv_fp8.dim() == 4 else kv_fp8
    if k8.dim() == 2:
        k8 = k8.unsqueeze(1)
    if k8.dim() != 3 or k8.shape[-1] != FP8_REC_BYTES:
        raise ValueError(f"kv_fp8 must be [S_kv, {FP8_REC_BYTES}] or [S_kv, G, {FP8_REC_BYTES}]")
    k8 = _prep(k8, torch.uint8, "kv_fp8", q3.device)
    G = k8.shape[1]
    ix = _grouped_idx(indices, G)
    if ix.dtype != torch.int32:
        ix = ix.to(torch.int32)
    ix = _prep(ix, torch.int32, "indices", q3.device)
    S, H, _ = q3.shape
    if ix.shape[0] != S:
        raise ValueError("indices must have one row per query token")
    K = ix.shape[2]
    S_kv = k8.shape[0]
    dev = q3.device
    if out is None:
        out = torch.empty(*lead[:-1], H, D_V, dtype=torch.bfloat16, device=dev)
    else:
        _dest(out, torch.bfloat16, S * H * D_V, dev, "out")
    if lse is None:
        lse = torch.empty(*lead[:-1], H, dtype=torch.float32, device=dev)
    else:
        _dest(lse, torch.float32, S * H, dev, "lse")
    ws, ws_addr = _workspace(fwd_workspace_bytes(S, S_kv, H, K, G), dev)
    flags = _lib.SMLA_FP8_POW2_SCALES if pow2_scales else 0
    _lib.check(lib.smla_fwd_fp8(_ptr(q3), _ptr(k8), _ptr(ix), S, S_kv, H, G, K, float(sm_scale),
                                _ptr(out), _ptr(lse), flags, ctypes.c_void_p(ws_addr),
                                ws.numel() - (ws_addr - ws.data_ptr()), _stream(dev)))
    return out, lse


def sparse_mla_bwd(q: torch.Tensor, kv: torch.Tensor, out: torch.Tensor, dout: torch.Tensor,
                   indices: torch.Tensor, lse: torch.Tensor, sm_scale: float, *,
                   dkv_f32: torch.Tensor | None = None, accumulate: bool = False,
                   atomic: bool = False, stored_p: bool = False,
                   want_bf16_dkv: bool = True):
    """Backward: returns (dq like q, dkv like kv in bf16 or None).

    kv and indices take the shapes sparse_mla_fwd takes (with or without a KV
    group dimension); dkv has kv's shape.  dkv_f32, if given, is a contiguous
    fp32 tensor of kv's element count that receives the fp32 dkv
    (overwritten, or added to with accumulate=True).  The default mode is
    the deterministic per-row reduction; atomic=True scatters dkv with fp32
    atomic adds (not bitwise reproducible).  stored_p=True has the dq pass
    store P and scale * dS for the dkv pass (one recompute of the scores
    instead of two; a larger workspace)."""
    lib = _lib.load()
    q3 = _prep(_flat_q(q), torch.bfloat16, "q")
    kv3, G = _grouped_kv(kv)
    kv3 = _prep(kv3, torch.bfloat16, "kv", q3.device)
    S, H, _ = q3.shape
    for name, t, n in (("out", out, S * H * D_V), ("dout", dout, S * H * D_V), ("lse", lse, S * H)):
        if t.numel() != n:
            raise ValueError(f"{name} must hold {n} elements, got {t.numel()}")
    o3 = _prep(out.reshape(S, H, D_V), torch.bfloat16, "out", q3.device)
    do3 = _prep(dout.reshape(S, H, D_V), torch.bfloat16, "dout", q3.device)
    ls = _prep(lse.reshape(S, H), torch.float32, "lse", q3.device)
    ix = _grouped_idx(indices, G)
    if ix.dtype != torch.int32:
        ix = ix.to(torch.int32)
    ix = _prep(ix, torch.int32, "indices", q3.device)
    if ix.shape[0] != S:
        raise ValueError("indices must have one row per query token")
    K = ix.shape[2]
    S_kv = kv3.shape[0]
    dev = q3.device
    flags = (_lib.SMLA_DKV_ATOMIC if atomic else 0) | (_lib.SMLA_DKV_STORED_P if stored_p else 0)
    if accumulate:
        if dkv_f32 is None:
            raise ValueError("accumulate=True needs dkv_f32")
        flags |= _lib.SMLA_DKV_ACCUMULATE
    if dkv_f32 is not None:
        _dest(dkv_f32, torch.float32, S_kv * G * D_K, dev, "dkv_f32")
    dq = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    dkv = torch.empty(kv.shape, dtype=torch.bfloat16, device=dev) if want_bf16_dkv else None
    ws, ws_addr = _workspace(bwd_workspace_bytes(S, S_kv, H, K, flags, G), dev)
    _lib.check(lib.smla_bwd_g(_ptr(q3), _ptr(kv3), _ptr(o3), _ptr(do3), _ptr(ix), _ptr(ls),
                              S, S_kv, H, G, K, float(sm_scale), _ptr(dq), _ptr(dkv),
                              _ptr(dkv_f32), flags, ctypes.c_void_p(ws_addr),
                              ws.numel() - (ws_addr - ws.data_ptr()), _stream(dev)))
    return dq, dkv


def validate_indices(indices: torch.Tensor, s_kv: int) -> int:
    """Number of index entries that are neither -1 nor in [0, s_kv).
    (Synchronizes the current stream to read the count.)"""
    lib = _lib.load()
    ix = indices.reshape(-1, indices.shape[-1])   # [S, K], [S, G, K] or [1, S, G, K]
    if ix.dtype != torch.int32:
        ix = ix.to(torch.int32)
    ix = _prep(ix, torch.int32, "indices")
    cnt = torch.empty(1, dtype=torch.int64, device=ix.device)
    _lib.check(lib.smla_validate_indices(_ptr(ix), ix.shape[0], ix.shape[1], s_kv, _ptr(cnt),
                                         _stream(ix.device)))
    return int(cnt.item())


def topk_indices(logits: torch.Tensor, ks: torch.Tensor, ke: torch.Tensor, topk: int,
                 out: torch.Tensor | None = None) -> torch.Tensor:
    """Index production: int32 [S, topk] top-k kv positions of each query's
    fp32 indexer logits [S, S_kv] inside its range [ks, ke), k capped at the
    range length, ascending, padded with -1 (the layout sparse_mla_fwd takes)."""
    lib = _lib.load()
    if (not _on_device(logits, None) or logits.dim() != 2 or logits.dtype != torch.float32
            or logits.stride(1) != 1):
        raise ValueError("logits must be an fp32 GPU tensor [S, S_kv] with contiguous rows")
    S, S_kv = logits.shape
    ks = _prep(ks.to(torch.int32), torch.int32, "ks", logits.device)
    ke = _prep(ke.to(torch.int32), torch.int32, "ke", logits.device)
    if ks.shape != (S,) or ke.shape != (S,):
        raise ValueError("ks and ke must be [S]")
    if out is None:
        out = torch.empty(S, topk, dtype=torch.int32, device=logits.device)
    else:
        _dest(out, torch.int32, S * topk, logits.device, "out")
    _lib.check(lib.smla_topk_indices(_ptr(logits), S, S_kv, logits.stride(0), _ptr(ks), _ptr(ke),
                                     topk, _ptr(out), _stream(logits.device)))
    return out


_DIAG_DTYPES = {torch.bfloat16: _lib.SMLA_DTYPE_BF16, torch.float32: _lib.SMLA_DTYPE_F32}


def _diag_operand(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype not in _DIAG_DTYPES:
        raise TypeError(f"{name} must be bf16 or fp32, got {t.dtype}")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    return t


def _counter(counter: torch.Tensor | None, device) -> torch.Tensor:
    if counter is None:
        return torch.zeros(1, dtype=torch.int64, device=device)
    if counter.dtype != torch.int64 or counter.numel() < 1 or not counter.is_cuda:
        raise ValueError("counter must be an int64 GPU tensor")
    return counter


def count_nonfinite(t: torch.Tensor, counter: torch.Tensor | None = None) -> int | None:
    """Number of NaN / Inf entries of a contiguous bf16 or fp32 GPU tensor.
    With `counter` (an int64 GPU tensor), the count is added into counter[0]
    without synchronizing and None is returned; without it, the call waits
    for the count and returns it."""
    lib = _lib.load()
    t = _diag_operand(t, "t")
    c = _counter(counter, t.device)
    _lib.check(lib.smla_nonfinite_count(_ptr(t), _DIAG_DTYPES[t.dtype], t.numel(), _ptr(c),
                                        _stream(t.device)))
    return None if counter is not None else int(c.item())


def replace_nonfinite_(t: torch.Tensor, ref: torch.Tensor | None = None,
                       counter: torch.Tensor | None = None) -> int | None:
    """In place: every NaN / Inf entry of `t` takes the value of the same
    entry of `ref` (zero when ref is None); other entries are untouched.
    Returns the number replaced (or adds it into `counter`, as in
    count_nonfinite)."""
    lib = _lib.load()
    t = _diag_operand(t, "t")
    if ref is not None:
        ref = _diag_operand(ref, "ref")
        if ref.dtype != t.dtype or ref.shape != t.shape:
            raise ValueError("ref must match t in dtype and shape")
    c = _counter(counter, t.device)
    _lib.check(lib.smla_nonfinite_replace(_ptr(t), _ptr(ref), _DIAG_DTYPES[t.dtype], t.numel(),
                                          _ptr(c), _stream(t.device)))
    return None if counter is not None else int(c.item())


class NonfiniteGradientError(RuntimeError):
    """sparse_mla_bwd_checked found NaN / Inf in dq or dkv."""


def sparse_mla_bwd_checked(q, kv, out, dout, indices, lse, sm_scale, reference=None,
                           on_nonfinite: str = "raise"):
    """The backward with the finite check of the pages' fallback workflow:
    run sparse_mla_bwd, count NaN / Inf in dq and dkv on the device (one read
    back for both), and if there are any, either take the values of a
    caller-supplied `reference(q, kv, out, dout, indices, lse, sm_scale) ->
    (dq_ref, dkv_ref)` at those entries only, or (no reference) raise
    NonfiniteGradientError (on_nonfinite="raise") or write zeros there
    (on_nonfinite="zero", a diagnostic confinement, not a fix).
    Returns (dq, dkv, {"dq": n, "dkv": n, "replaced": n})."""
    if on_nonfinite not in ("raise", "zero"):
        raise ValueError("on_nonfinite must be 'raise' or 'zero'")
    dq, dkv = sparse_mla_bwd(q, kv, out, dout, indices, lse, sm_scale)
    cnt = torch.zeros(2, dtype=torch.int64, device=dq.device)
    count_nonfinite(dq, cnt[0:1])
    count_nonfinite(dkv, cnt[1:2])
    n_dq, n_dkv = (int(v) for v in cnt.tolist())
    info = {"dq": n_dq, "dkv": n_dkv, "replaced": 0}
    if n_dq + n_dkv == 0:
        return dq, dkv, info
    if reference is not None:
        dq_ref, dkv_ref = reference(q, kv, out, dout, indices, lse, sm_scale)
        dq_ref = dq_ref.to(dq.dtype).reshape(dq.shape).contiguous()
        dkv_ref = dkv_ref.to(dkv.dtype).reshape(dkv.shape).contiguous()
    elif on_nonfinite == "raise":
        raise NonfiniteGradientError(f"nonfinite entries: dq {n_dq}, dkv {n_dkv}")
    else:
        dq_ref = dkv_ref = None
    info["replaced"] = replace_nonfinite_(dq, dq_ref) + replace_nonfinite_(dkv, dkv_ref)
    return dq, dkv, info


class SparseMLA(torch.autograd.Function):
    """out = SparseMLA.apply(q, kv, indices, sm_scale): differentiable in q and kv."""

    @staticmethod
    def forward(ctx, q, kv, indices, sm_scale):
        out, lse = sparse_mla_fwd(q, kv, indices, sm_scale)
        ctx.save_for_backward(q, kv, indices, out, lse)
        ctx.sm_scale = sm_scale
        return out

    @staticmethod
    def backward(ctx, grad_out):
        q, kv, indices, out, lse = ctx.saved_tensors
        dq, dkv = sparse_mla_bwd(q, kv, out, grad_out.contiguous(), indices, lse, ctx.sm_scale)
        return dq, dkv, None, None


class SparseMLARunner:
    """Repeated forward + backward on fixed shapes with every buffer
    preallocated: each call enqueues the library's kernels and allocates
    nothing.  Inputs must already be contiguous bf16/int32 GPU tensors of the
    shapes given here: with kv_groups = G > 1, kv [s_kv, G, 576] and indices
    [s_q, G, topk] (dkv like kv)."""

    def __init__(self, s_q: int, s_kv: int, heads: int, topk: int, device="cuda",
                 dkv_atomic: bool = False, dkv_stored_p: bool = False, kv_groups: int = 1):
        self.lib = _lib.load()
        self.shape = (s_q, s_kv, heads, topk)
        self.G = kv_groups
        kv_shape = (s_kv, D_K) if kv_groups == 1 else (s_kv, kv_groups, D_K)
        self._kv_shape = kv_shape
        self._idx_shape = (s_q, topk) if kv_groups == 1 else (s_q, kv_groups, topk)
        self._bflags = ((_lib.SMLA_DKV_ATOMIC if dkv_atomic else 0) |
                        (_lib.SMLA_DKV_STORED_P if dkv_stored_p else 0))
        dev = torch.device(device)
        self.out = torch.empty(s_q, heads, D_V, dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty(s_q, heads, dtype=torch.float32, device=dev)
        self.dq = torch.empty(s_q, heads, D_K, dtype=torch.bfloat16, device=dev)
        self.dkv = torch.empty(*kv_shape, dtype=torch.bfloat16, device=dev)
        fb = fwd_workspace_bytes(s_q, s_kv, heads, topk, kv_groups)
        bb = bwd_workspace_bytes(s_q, s_kv, heads, topk, self._bflags, kv_groups)
        self._fws, self._fws_addr = _workspace(fb, dev)
        self._bws, self._bws_addr = _workspace(bb, dev)
        self._fb, self._bb = fb, bb
        self.device = dev

    def _check(self, q=None, kv=None, idx=None, dout=None):
        """Shapes, dtypes and layouts of the given inputs against the runner's
        (host-side only: no synchronization); raises ValueError."""
        s_q, s_kv, h, k = self.shape
        want = (("q", q, (s_q, h, D_K), torch.bfloat16), ("kv", kv, self._kv_shape, torch.bfloat16),
                ("indices", idx, self._idx_shape, torch.int32),
                ("dout", dout, (s_q, h, D_V), torch.bfloat16))
        for name, t, shape, dtype in want:
            if t is None:
                continue
            if tuple(t.shape) != shape or t.dtype != dtype or not t.is_contiguous() or not t.is_cuda:
                raise ValueError(f"{name} must be a contiguous {dtype} GPU tensor of shape {shape}")

    def plan(self, idx):
        """Build the index plan once (smla_plan) into the backward workspace;
        fwd / bwd with planned=True then reuse it (same indices)."""
        s_q, s_kv, h, k = self.shape
        self._check(idx=idx)
        _lib.check(self.lib.smla_plan_g(_ptr(idx), s_q, s_kv, h, self.G, k,
                                        ctypes.c_void_p(self._bws_addr), self._bb,
                                        _stream(self.device)))

    def fwd(self, q, kv, idx, sm_scale, planned: bool = False):
        s_q, s_kv, h, k = self.shape
        self._check(q, kv, idx)
        ws, wb = (self._bws_addr, self._bb) if planned else (self._fws_addr, self._fb)
        _lib.check(self.lib.smla_fwd_g(_ptr(q), _ptr(kv), _ptr(idx), s_q, s_kv, h, self.G, k,
                                       float(sm_scale), _ptr(self.out), _ptr(self.lse),
                                       _lib.SMLA_PLAN_READY if planned else 0, ctypes.c_void_p(ws),
                                       wb, _stream(self.device)))
        return self.out, self.lse

    def fwd_fp8(self, q, kv_fp8, idx, sm_scale, planned: bool = False,
                pow2_scales: bool = False):
        """The forward over fp8 kv records (uint8 [s_kv, 656], or [s_kv, G,
        656]) into the runner's out / lse (pow2_scales as in
        sparse_mla_fwd_fp8)."""
        s_q, s_kv, h, k = self.shape
        self._check(q=q, idx=idx)
        if (kv_fp8.dtype != torch.uint8 or not kv_fp8.is_cuda or not kv_fp8.is_contiguous()
                or kv_fp8.numel() != s_kv * self.G * FP8_REC_BYTES):
            raise ValueError(f"kv_fp8 must be a contiguous uint8 GPU tensor of "
                             f"s_kv * kv_groups * {FP8_REC_BYTES} bytes")
        ws, wb = (self._bws_addr, self._bb) if planned else (self._fws_addr, self._fb)
        flags = ((_lib.SMLA_PLAN_READY if planned else 0) |
                 (_lib.SMLA_FP8_POW2_SCALES if pow2_scales else 0))
        _lib.check(self.lib.smla_fwd_fp8(_ptr(q), _ptr(kv_fp8), _ptr(idx), s_q, s_kv, h, self.G, k,
                                         float(sm_scale), _ptr(self.out), _ptr(self.lse),
                                         flags,
                                         ctypes.c_void_p(ws), wb, _stream(self.device)))
        return self.out, self.lse

    def bwd(self, q, kv, dout, idx, sm_scale, planned: bool = False):
        s_q, s_kv, h, k = self.shape
        self._check(q, kv, idx, dout)
        _lib.check(self.lib.smla_bwd_g(_ptr(q), _ptr(kv), _ptr(self.out), _ptr(dout), _ptr(idx),
                                       _ptr(self.lse), s_q, s_kv, h, self.G, k, float(sm_scale),
                                       _ptr(self.dq), _ptr(self.dkv), ctypes.c_void_p(0),
                                       self._bflags | (_lib.SMLA_PLAN_READY if planned else 0),
                                       ctypes.c_void_p(self._bws_addr), self._bb,
                                       _stream(self.device)))
        return self.dq, self.dkv


def timing_start(max_launches: int) -> None:
    """Bracket every kernel the library launches with HIP events (benchmarks)."""
    _lib.check(_lib.load().smla_timing_start(max_launches))


def timing_stop() -> None:
    _lib.check(_lib.load().smla_timing_stop())


def timing_read(kernel: str) -> tuple[int, float]:
    """(launches recorded, total milliseconds) for one kernel name."""
    n = ctypes.c_int(0)
    ms = ctypes.c_double(0.0)
    _lib.check(_lib.load().smla_timing_read(kernel.encode(), ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value
