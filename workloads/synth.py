"""Seeded synthetic inputs for sparse-MLA attention (DSA, absorbed-latent layout).

This module only draws inputs. It holds none of the attention arithmetic, so
both the fp64 oracle's tests and the HIP path's tests and benchmark may use it.

Layout of everything returned (packed "thd" layout, one KV group):
  q      [S, H, 576]  bf16 bits (uint16)   absorbed-latent query, 512 latent + 64 rope
  kv     [S_kv, 576]  bf16 bits (uint16)   shared latent KV; value = columns 0:512
  dout   [S, H, 512]  bf16 bits (uint16)   upstream gradient of out
  idx    [S, K]       int32                absolute rows of kv; -1 marks padding

The index structure follows the production workload the pages describe: the
forward/backward fix of miles PR #2079 ("fix GLM-5 sparse-MLA kernel -1 index
OOB and NaN gradients", section 实现拆解 item 4) was checked at H=8, topk=2048
on ragged packed sequences including all -1 rows, and the -1 sentinel comes
from padding a capped top-k back to the fixed width (Megatron-Bridge PR #17,
"GLM-5 DSA option: tilelang (2/2)", section Bug fixes).

Draw order for every workload: q, kv, dout as fp32 standard normals (times the
workload's sigma) rounded to bf16 with round-to-nearest-even; then sequence
lengths (where drawn); then indices; then the rows that are emptied or scaled.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

D_LATENT = 512
D_ROPE = 64
D_QK = D_LATENT + D_ROPE
SM_SCALE = 1.0 / math.sqrt(192.0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return the bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1).view(np.uint32)
    out = np.empty(flat.shape, dtype=np.uint16)
    step = 1 << 24
    for i in range(0, flat.size, step):           # bounded temporaries on large tensors
        b = flat[i:i + step].astype(np.uint64)
        rounding = np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))
        out[i:i + step] = ((b + rounding) >> np.uint64(16)).astype(np.uint16)
    return out.reshape(x.shape)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float64."""
    return bf16_bits_to_f32(bits).astype(np.float64)


@dataclass
class Workload:
    name: str
    q: np.ndarray          # uint16 [S, H, 576]
    kv: np.ndarray         # uint16 [S_kv, 576]
    dout: np.ndarray       # uint16 [S, H, 512]
    idx: np.ndarray        # int32 [S, K]
    sm_scale: float
    seqlens: list = field(default_factory=list)
    seed: int = 0

    @property
    def S(self) -> int:
        return self.q.shape[0]

    @property
    def H(self) -> int:
        return self.q.shape[1]

    @property
    def S_kv(self) -> int:
        return self.kv.shape[0]

    @property
    def K(self) -> int:
        return self.idx.shape[1]

    @property
    def n_valid(self) -> int:
        """Number of valid (token, slot) pairs: slots holding a row in [0, S_kv)."""
        return int(np.count_nonzero((self.idx >= 0) & (self.idx < self.S_kv)))


_CHUNK = 1 << 22   # values per independently seeded chunk of a large tensor


def _normal_bf16(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    """N(0, sigma^2) values rounded to bf16.  The tensor is cut into chunks of
    _CHUNK values, each drawn from its own generator seeded from `rng` (so the
    result depends only on the seed), generated on a few threads."""
    n = int(np.prod(shape))
    nchunk = (n + _CHUNK - 1) // _CHUNK
    seeds = rng.integers(0, 2**63 - 1, size=nchunk, dtype=np.int64)
    out = np.empty(n, dtype=np.uint16)

    def work(i):
        g = np.random.default_rng(int(seeds[i]))
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        x = g.standard_normal(size=hi - lo, dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        out[lo:hi] = f32_to_bf16_bits(x)

    if nchunk == 1:
        work(0)
    else:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=min(8, nchunk)) as ex:
            list(ex.map(work, range(nchunk)))
    return out.reshape(shape)


def _tensors(rng, S, H, S_kv, sigma=1.0):
    q = _normal_bf16(rng, (S, H, D_QK), sigma)
    kv = _normal_bf16(rng, (S_kv, D_QK), sigma)
    dout = _normal_bf16(rng, (S, H, D_LATENT), 1.0)
    return q, kv, dout


def _starts(seqlens):
    return np.concatenate([[0], np.cumsum(seqlens)[:-1]]).astype(np.int64)


def causal_full_rows(rng, seqlens, K) -> np.ndarray:
    """Row p of each sequence lists all p+1 in-sequence causal positions, in a
    random order, followed by -1; positions beyond K are not possible here, so
    every sequence length must be <= K."""
    S = int(sum(seqlens))
    idx = np.full((S, K), -1, dtype=np.int32)
    for start, n in zip(_starts(seqlens), seqlens):
        assert n <= K, "full causal rows need seqlen <= topk"
        for p in range(n):
            row = rng.permutation(p + 1).astype(np.int32) + np.int32(start)
            idx[start + p, : p + 1] = row
    return idx


def _uniform_picks(rng, cand: np.ndarray, k: int, batch: int = 256) -> np.ndarray:
    """Row i: min(k, cand[i]) distinct values of range(cand[i]) drawn uniformly,
    in random order, then -1.  Random-key sampling: every candidate gets an
    independent uniform key, the k smallest keys are kept, in key order."""
    n = len(cand)
    out = np.full((n, k), -1, dtype=np.int64)
    for b in range(0, n, batch):
        c = np.asarray(cand[b:b + batch], dtype=np.int64)
        m = int(c.max()) if c.size else 0
        if m == 0:
            continue
        keys = rng.random((len(c), m))
        keys[np.arange(m)[None, :] >= c[:, None]] = np.inf
        kk = min(k, m)
        part = np.argpartition(keys, kk - 1, axis=1)[:, :kk]
        pk = np.take_along_axis(keys, part, 1)
        order = np.argsort(pk, axis=1)
        sel = np.take_along_axis(part, order, 1)
        ok = np.take_along_axis(pk, order, 1) < np.inf
        out[b:b + len(c), :kk] = np.where(ok, sel, -1)
    return out


def causal_uniform_rows(rng, seqlens, K) -> np.ndarray:
    """Row p picks min(K, p+1) distinct causal in-sequence positions uniformly
    (in random order); the rest of the row is -1."""
    S = int(sum(seqlens))
    idx = np.full((S, K), -1, dtype=np.int32)
    for start, n in zip(_starts(seqlens), seqlens):
        picks = _uniform_picks(rng, np.arange(1, n + 1), K)
        idx[start:start + n] = np.where(picks >= 0, picks + start, -1).astype(np.int32)
    return idx


def causal_recency_rows(rng, seqlens, K, recent=512) -> np.ndarray:
    """Rows with at least K candidates take every one of the last `recent`
    positions plus K-`recent` distinct uniform picks from the older positions
    (all in random order); shorter rows list every causal position.  (One
    reading of "half the picks from the last 512 positions": half of K=2048
    cannot be met with distinct picks out of 512 positions, so all 512 are
    taken and the rest are uniform.)"""
    S = int(sum(seqlens))
    idx = np.full((S, K), -1, dtype=np.int32)
    for start, n in zip(_starts(seqlens), seqlens):
        cand = np.arange(1, n + 1)
        short = cand <= K
        rows = np.full((n, K), -1, dtype=np.int64)
        rows[short] = _uniform_picks(rng, cand[short], K)
        longr = np.nonzero(~short)[0]
        if longr.size:
            old = _uniform_picks(rng, cand[longr] - recent, K - recent)
            recent_rows = (cand[longr] - recent)[:, None] + np.arange(recent)[None, :]
            full = np.concatenate([recent_rows, old], axis=1)
            perm = np.argsort(rng.random(full.shape), axis=1)
            rows[longr] = np.take_along_axis(full, perm, 1)
        idx[start:start + n] = np.where(rows >= 0, rows + start, -1).astype(np.int32)
    return idx


def ragged_lengths(rng, n_seq, lo, hi, total) -> list:
    """n_seq lengths drawn uniformly in [lo, hi], then nudged by +-1 steps on
    randomly chosen sequences (staying inside [lo, hi]) until they sum to total."""
    lens = rng.integers(lo, hi + 1, size=n_seq).astype(np.int64)
    assert n_seq * lo <= total <= n_seq * hi
    while lens.sum() != total:
        i = int(rng.integers(0, n_seq))
        if lens.sum() < total and lens[i] < hi:
            lens[i] += 1
        elif lens.sum() > total and lens[i] > lo:
            lens[i] -= 1
    return [int(x) for x in lens]


# ---------------------------------------------------------------------------
# The five workloads.  Each is named by what it is; the seeds are 0..4.
# ---------------------------------------------------------------------------

def tiny(seed: int = 0) -> Workload:
    """S=128 single sequence, H=8, topk=64; row s holds min(64, s+1) distinct
    causal positions drawn uniformly, padded with -1."""
    rng = np.random.default_rng(seed)
    S, H, K = 128, 8, 64
    q, kv, dout = _tensors(rng, S, H, S)
    idx = causal_uniform_rows(rng, [S], K)
    return Workload("tiny_s128_h8_k64", q, kv, dout, idx, SM_SCALE, [S], seed)


def packed_ragged(seed: int = 1) -> Workload:
    """S=4096 packed as sequences {512, 1024, 1536, 1024}, H=8, topk=2048.
    Every length is below topk, so row p lists all p+1 in-sequence causal
    positions (shuffled) followed by 2047-p trailing -1."""
    rng = np.random.default_rng(seed)
    seqlens = [512, 1024, 1536, 1024]
    S, H, K = sum(seqlens), 8, 2048
    q, kv, dout = _tensors(rng, S, H, S)
    idx = causal_full_rows(rng, seqlens, K)
    return Workload("packed_ragged_s4096_h8_k2048", q, kv, dout, idx, SM_SCALE, seqlens, seed)


def repeated_slots(seed: int = 6, dup_frac: float = 0.001) -> Workload:
    """The packed ragged batch with a fraction `dup_frac` of the valid slots
    overwritten by a copy of another valid slot of the same row, so some rows
    list a kv row twice (each slot stays its own softmax term): the input
    class that takes the planner's and the dkv finalize's repeated-slot path."""
    w = packed_ragged(seed)
    rng = np.random.default_rng(seed + 100)
    idx = w.idx.copy()
    for s in range(w.S):
        nv = int((idx[s] >= 0).sum())
        if nv < 2:
            continue
        m = np.nonzero(rng.random(nv) < dup_frac)[0]
        if m.size:
            src = rng.integers(0, nv, size=m.size)
            idx[s, m] = idx[s, src]
    return Workload(f"repeated_slots_s{w.S}_h{w.H}_k{w.K}_dup{dup_frac:g}", w.q, w.kv, w.dout, idx,
                    SM_SCALE, w.seqlens, seed)


def padding_stress(seed: int = 2, sigma: float = 2.0) -> Workload:
    """S=4096 packed as 16 sequences with lengths uniform in [16, 512] (nudged to
    sum to 4096), H=8, topk=2048, q/kv ~ N(0, sigma^2) with sigma=2 (variance 4)
    for large logits; full causal rows, then 5% of the rows set entirely to -1."""
    rng = np.random.default_rng(seed)
    S, H, K = 4096, 8, 2048
    q, kv, dout = _tensors(rng, S, H, S, sigma=sigma)
    seqlens = ragged_lengths(rng, 16, 16, 512, S)
    idx = causal_full_rows(rng, seqlens, K)
    n_empty = int(round(0.05 * S))
    empty = rng.choice(S, size=n_empty, replace=False)
    idx[empty, :] = -1
    return Workload(f"padding_stress_s4096_h8_k2048_sigma{sigma:g}", q, kv, dout, idx,
                    SM_SCALE, seqlens, seed)


def recency_hot_rows(seed: int = 3) -> Workload:
    """Single sequence S=8192, H=16, topk=2048 with a recency bias: every row
    with more than 2048 candidates takes all of its last 512 positions plus
    1536 uniform picks from the older ones (hot KV rows, dKV contention)."""
    rng = np.random.default_rng(seed)
    S, H, K = 8192, 16, 2048
    q, kv, dout = _tensors(rng, S, H, S)
    idx = causal_recency_rows(rng, [S], K)
    return Workload("recency_s8192_h16_k2048", q, kv, dout, idx, SM_SCALE, [S], seed)


def long_context(seed: int = 4) -> Workload:
    """S=32768 packed as 2 x 16384, H=16, topk=2048 uniform distinct causal
    picks; 1% of the kv rows (seeded) are drawn with 30x the scale."""
    rng = np.random.default_rng(seed)
    seqlens = [16384, 16384]
    S, H, K = sum(seqlens), 16, 2048
    q = _normal_bf16(rng, (S, H, D_QK), 1.0)
    kv32 = rng.standard_normal(size=(S, D_QK), dtype=np.float32)
    dout = _normal_bf16(rng, (S, H, D_LATENT), 1.0)
    idx = causal_uniform_rows(rng, seqlens, K)
    hot = rng.choice(S, size=int(round(0.01 * S)), replace=False)
    kv32[hot] *= np.float32(30.0)
    kv = f32_to_bf16_bits(kv32)
    return Workload("long_context_s32768_h16_k2048", q, kv, dout, idx, SM_SCALE, seqlens, seed)


def heads128(seed: int = 5) -> Workload:
    """S=2048 packed as sequences {512, 1536}, H=128 (one GPU's query heads
    with no head split), topk=2048; row p lists all p+1 in-sequence causal
    positions (shuffled) followed by trailing -1."""
    rng = np.random.default_rng(seed)
    seqlens = [512, 1536]
    S, H, K = sum(seqlens), 128, 2048
    q, kv, dout = _tensors(rng, S, H, S)
    idx = causal_full_rows(rng, seqlens, K)
    return Workload("packed_ragged_s2048_h128_k2048", q, kv, dout, idx, SM_SCALE, seqlens, seed)


WORKLOADS = {
    "tiny": tiny,
    "packed_ragged": packed_ragged,
    "padding_stress": padding_stress,
    "recency": recency_hot_rows,
    "long_context": long_context,
    "heads128": heads128,
    "repeated_slots": repeated_slots,
}


@dataclass
class GroupedWorkload:
    """Inputs with G kv groups: q [S, H, 576], kv [S_kv, G, 576], dout
    [S, H, 512] (bf16 bits) and idx [S, G, K] int32; heads g H/G .. (g+1) H/G - 1
    use kv group g and index rows idx[:, g]."""
    q: np.ndarray
    kv: np.ndarray
    dout: np.ndarray
    idx: np.ndarray
    sm_scale: float

    @property
    def S(self) -> int:
        return self.q.shape[0]

    @property
    def H(self) -> int:
        return self.q.shape[1]

    @property
    def G(self) -> int:
        return self.kv.shape[1]

    @property
    def S_kv(self) -> int:
        return self.kv.shape[0]

    @property
    def K(self) -> int:
        return self.idx.shape[2]


def custom_grouped(S, H, G, K, S_kv, seed=0, **kw) -> GroupedWorkload:
    """custom() per kv group (seeds seed * 64 + g), stacked: group g's heads,
    kv rows and index rows are those of its own custom() draw."""
    parts = [custom(S, H // G, K, S_kv, seed=seed * 64 + g, **kw) for g in range(G)]
    return GroupedWorkload(q=np.concatenate([p.q for p in parts], axis=1),
                           kv=np.stack([p.kv for p in parts], axis=1),
                           dout=np.concatenate([p.dout for p in parts], axis=1),
                           idx=np.stack([p.idx for p in parts], axis=1),
                           sm_scale=parts[0].sm_scale)


FP8_REC_BYTES = 656   # e4m3 latent [512], fp32 scales [4], bf16 rope [64]


def quantize_kv_fp8(kv_bits: np.ndarray, pow2_scales: bool = True) -> np.ndarray:
    """fp8 kv records [..., 656] (uint8) of bf16 kv rows [..., 576] (bits):
    per row and 128-column block of the latent part, scale = amax / 448
    (rounded up to a power of two with pow2_scales, so that every decoded
    value is exact in bf16; 1 for an all-zero block) and codes = e4m3 (OCP,
    round to nearest even) of value / scale; the rope columns keep their bf16
    bits.  Input encoding for the fp8 forward's tests and bench."""
    import torch
    bits = np.ascontiguousarray(kv_bits, dtype=np.uint16)
    lead = bits.shape[:-1]
    flat = bits.reshape(-1, 576)
    x = bf16_bits_to_f32(flat[:, :512]).reshape(-1, 4, 128)
    amax = np.abs(x).max(axis=2)
    scale = np.where(amax > 0, amax / 448.0, 1.0).astype(np.float32)
    if pow2_scales:
        scale = np.exp2(np.ceil(np.log2(scale))).astype(np.float32)
    y = np.clip(x / scale[:, :, None], -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(y.reshape(-1, 512)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    rec = np.zeros((flat.shape[0], FP8_REC_BYTES), dtype=np.uint8)
    rec[:, :512] = codes
    rec[:, 512:528] = scale.astype("<f4").view(np.uint8).reshape(-1, 16)
    rec[:, 528:] = flat[:, 512:].astype("<u2").view(np.uint8).reshape(-1, 128)
    return rec.reshape(*lead, FP8_REC_BYTES)


def causal_ranges(seqlens):
    """Key ranges [ks, ke) of packed causal sequences (input structure for the
    index-production step): token p of a sequence starting at row c sees kv
    rows c .. c + p."""
    ks, ke, c = [], [], 0
    for L in seqlens:
        ks.extend([c] * int(L))
        ke.extend(range(c + 1, c + int(L) + 1))
        c += int(L)
    return np.asarray(ks, dtype=np.int32), np.asarray(ke, dtype=np.int32)


def custom(S, H, K, S_kv=None, seed=0, sigma=1.0, pad_frac=0.3, empty_frac=0.1,
           dup_frac=0.0, scatter_pad=True, oob_frac=0.0) -> Workload:
    """Small free-form workload for edge-case tests: random rows of kv (not
    causal), a fraction of slots set to -1 at random positions (or trailing),
    some rows entirely -1, optional duplicate entries, optional out-of-range
    entries (values >= S_kv or < -1) for the safety tests."""
    rng = np.random.default_rng(seed)
    S_kv = S if S_kv is None else S_kv
    q, kv, dout = _tensors(rng, S, H, S_kv, sigma=sigma)
    idx = np.empty((S, K), dtype=np.int32)
    for s in range(S):
        if K <= S_kv:
            idx[s] = rng.choice(S_kv, size=K, replace=False)
        else:
            idx[s] = rng.integers(0, S_kv, size=K)
    if dup_frac > 0:
        m = rng.random((S, K)) < dup_frac
        src = rng.integers(0, K, size=(S, K))
        idx[m] = idx[np.nonzero(m)[0], src[m]]
    if pad_frac > 0:
        if scatter_pad:
            idx[rng.random((S, K)) < pad_frac] = -1
        else:
            n_pad = int(round(pad_frac * K))
            if n_pad:
                idx[:, K - n_pad:] = -1
    if empty_frac > 0:
        n_e = max(1, int(round(empty_frac * S)))
        idx[rng.choice(S, size=min(S, n_e), replace=False)] = -1
    if oob_frac > 0:
        m = rng.random((S, K)) < oob_frac
        bad = np.where(rng.random((S, K)) < 0.5, S_kv + rng.integers(0, 1000, size=(S, K)),
                       -2 - rng.integers(0, 1000, size=(S, K)))
        idx[m] = bad[m].astype(np.int32)
    return Workload(f"custom_s{S}_h{H}_k{K}_skv{S_kv}_seed{seed}", q, kv, dout, idx,
                    SM_SCALE, [S], seed)


def planted_nonfinite(n: int, dtype: str, frac: float = 0.01, seed: int = 0):
    """Input for the nonfinite diagnostics: n finite normal values (bf16 or
    fp32 bits) with a seeded fraction replaced by NaN / Inf bit patterns of
    every kind (quiet and signalling NaN of both signs, +-Inf), and a finite
    reference of the same shape.  Returns (bits, ref_bits)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n).astype(np.float32)
    r = rng.standard_normal(n).astype(np.float32)
    if dtype == "bf16":
        bits, ref = f32_to_bf16_bits(x), f32_to_bf16_bits(r)
        specials = np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x7F81, 0xFFFF, 0x7FFF], dtype=np.uint16)
    elif dtype == "f32":
        bits, ref = x.view(np.uint32).copy(), r.view(np.uint32).copy()
        specials = np.array([0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00000, 0x7F800001,
                             0xFFFFFFFF, 0x7FFFFFFF], dtype=np.uint32)
    else:
        raise ValueError("dtype must be 'bf16' or 'f32'")
    k = int(round(frac * n))
    if k:
        pos = rng.choice(n, size=k, replace=False)
        bits[pos] = specials[rng.integers(0, len(specials), k)]
    return bits, ref
