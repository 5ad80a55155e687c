"""The seeded generators: determinism, bf16 rounding, and index structure."""
import numpy as np
import torch

from workloads import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 7,
                        np.array([0.0, -0.0, 1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -9, 65504.0],
                                 dtype=np.float32)])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_tiny_deterministic_and_structured():
    a, b = synth.tiny(), synth.tiny()
    for f in ("q", "kv", "dout", "idx"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    assert a.q.shape == (128, 8, 576) and a.kv.shape == (128, 576) and a.dout.shape == (128, 8, 512)
    assert a.idx.shape == (128, 64) and a.idx.dtype == np.int32
    assert a.n_valid == 6176
    for s in range(128):
        n = min(64, s + 1)
        row = a.idx[s]
        assert np.all(row[n:] == -1)
        v = row[:n]
        assert len(set(v.tolist())) == n and v.min() >= 0 and v.max() <= s


def test_packed_ragged_rows_are_full_causal_lists():
    w = synth.packed_ragged()
    assert w.n_valid == 2361344 and w.K == 2048 and w.H == 8
    starts = np.cumsum([0] + w.seqlens[:-1])
    for st, n in zip(starts, w.seqlens):
        for p in (0, 1, n // 2, n - 1):
            row = w.idx[st + p]
            assert np.array_equal(np.sort(row[: p + 1]), np.arange(st, st + p + 1))
            assert np.all(row[p + 1:] == -1)


def test_recency_rows_small():
    rng = np.random.default_rng(0)
    idx = synth.causal_recency_rows(rng, [300], 64, recent=16)
    for p in range(300):
        row = idx[p]
        v = row[row != -1]
        assert len(set(v.tolist())) == len(v) == min(64, p + 1)
        assert v.max() <= p
        if p + 1 > 64:
            assert set(range(p - 15, p + 1)) <= set(v.tolist())


def test_uniform_rows_small():
    rng = np.random.default_rng(1)
    idx = synth.causal_uniform_rows(rng, [50, 70], 32)
    for s in range(120):
        st = 0 if s < 50 else 50
        v = idx[s][idx[s] != -1]
        assert len(v) == min(32, s - st + 1) and len(set(v.tolist())) == len(v)
        assert v.min() >= st and v.max() <= s


def test_ragged_lengths_sum_and_bounds():
    rng = np.random.default_rng(2)
    lens = synth.ragged_lengths(rng, 16, 16, 512, 4096)
    assert sum(lens) == 4096 and min(lens) >= 16 and max(lens) <= 512


def test_custom_edge_case_knobs():
    w = synth.custom(S=50, H=2, K=20, S_kv=40, seed=1, dup_frac=0.2, oob_frac=0.05)
    assert ((w.idx >= 40) | (w.idx < -1)).any()
    assert (w.idx == -1).all(axis=1).any()
