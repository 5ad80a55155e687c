"""Pins of the fp8 kv decoding of the oracle, independent of its code:

  * e4m3 values fixed by the format's definition (1.0, the largest normal
    448, the smallest normal 2^-6, the smallest subnormal 2^-9, the largest
    subnormal 7/8 * 2^-6, signed zero, NaN codes);
  * every non-NaN code against torch's float8_e4m3fn conversion (a library
    routine of the same OCP format);
  * a hand-built record: per-block scales, rope bits, little-endian layout;
  * the input quantizer: decoded values within half an e4m3 step of the
    input, exact with power-of-two scales when representable;
  * the bf16 rounding of decoded rows: ties to even at hand-picked halfway
    points, and torch's float32 -> bfloat16 conversion on random values.
"""
import math

import numpy as np
import pytest

from oracle import decode_e4m3, decode_kv_records, round_bf16
from oracle.smla_oracle import OracleInputError
from workloads import synth


def test_e4m3_values_fixed_by_the_format():
    v = decode_e4m3(np.array([0x38, 0x7E, 0x08, 0x01, 0x07, 0xB8, 0x00, 0x80, 0x40, 0x3C],
                             dtype=np.uint8))
    assert list(v[:6]) == [1.0, 448.0, 2.0 ** -6, 2.0 ** -9, 7 / 8 * 2.0 ** -6, -1.0]
    assert v[6] == 0.0 and not math.copysign(1.0, v[6]) < 0
    assert v[7] == 0.0 and math.copysign(1.0, v[7]) < 0
    assert v[8] == 2.0 and v[9] == 1.5
    assert np.isnan(decode_e4m3(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


def test_every_code_against_torch_float8_e4m3fn():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = decode_e4m3(codes)
    finite = ~np.isnan(ref)
    assert finite.sum() == 254
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.signbit(got[finite]), np.signbit(ref[finite]))
    assert np.isnan(got[~finite]).all()


def test_hand_built_record():
    rec = np.zeros(656, dtype=np.uint8)
    rec[:512] = 0x38                                                # 1.0
    rec[5] = 0xC0                                                   # -2.0
    rec[512:528] = np.array([1.0, 2.0, 0.5, 4.0], dtype="<f4").view(np.uint8)
    rec[528:] = np.full(64, 0x4040, dtype="<u2").view(np.uint8)     # bf16 3.0
    rec[528:530] = np.array([0xBF80], dtype="<u2").view(np.uint8)   # bf16 -1.0
    kv = decode_kv_records(rec)
    want = np.concatenate([np.full(128, 1.0), np.full(128, 2.0), np.full(128, 0.5),
                           np.full(128, 4.0), np.full(64, 3.0)])
    want[5] = -2.0
    want[512] = -1.0
    assert kv.shape == (576,) and np.array_equal(kv, want)
    with pytest.raises(OracleInputError):
        decode_kv_records(np.zeros((3, 655), dtype=np.uint8))


@pytest.mark.parametrize("pow2", [True, False])
def test_quantizer_round_trip(pow2):
    w = synth.custom(S=2, H=8, K=4, S_kv=64, seed=3)
    rec = synth.quantize_kv_fp8(w.kv, pow2_scales=pow2)
    x = synth.bf16_bits_to_f64(w.kv)
    d = decode_kv_records(rec)
    assert np.array_equal(d[:, 512:], x[:, 512:])
    scales = rec[:, 512:528].copy().view("<f4").astype(np.float64)
    step = np.repeat(scales, 128, axis=1) * 2.0 ** -3 * np.maximum(
        np.exp2(np.floor(np.log2(np.maximum(np.abs(x[:, :512]) / np.repeat(scales, 128, axis=1),
                                            2.0 ** -6)))), 2.0 ** -6)
    # half an e4m3 step of value / scale, plus the fp32 rounding of value / scale
    assert np.all(np.abs(d[:, :512] - x[:, :512]) <= 0.5 * step + 2.0 ** -22 * np.abs(x[:, :512]))
    # decoded latent values are exact in bf16 with power-of-two scales
    if pow2:
        b = synth.bf16_bits_to_f64(synth.f32_to_bf16_bits(d[:, :512].astype(np.float32)))
        assert np.array_equal(b, d[:, :512])


def test_bf16_rounding_ties_to_even():
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20, -(1 + 2.0 ** -8),
                  2.0 ** -130, 3.0])
    want = np.array([1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -1.0, 2.0 ** -130, 3.0])
    assert np.array_equal(round_bf16(x), want)


def test_bf16_rounding_against_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-20, 20, 20000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(round_bf16(x.astype(np.float64)), ref)
