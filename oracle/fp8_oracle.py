"""fp64 CPU oracle for the fp8 kv forward (test infrastructure only).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline may import or run this module; it shares no code with the HIP
library.

An fp8 kv row is a record of 656 bytes: the 512 latent columns as e4m3 codes,
four little-endian fp32 scales (scale b multiplies columns 128b .. 128b+127),
then the 64 rope columns as bf16.  The sources mention fp8 only as a serving
format (Megatron-Bridge / miles digests); the record layout is this library's
reading.  Decoding is exact in fp64:

  e4m3 (the OCP 8-bit format with 4 exponent bits, bias 7, 3 mantissa bits,
  no infinities): code = s eeee mmm
      eeee = 0:               (-1)^s * (m / 8) * 2^(1 - 7)     (subnormal)
      eeee = 15 and mmm = 7:  NaN
      otherwise:              (-1)^s * (1 + m / 8) * 2^(eeee - 7)
  latent value = decode(code) * scale;  rope value = the bf16 value.

The rows enter the attention as bf16, as every kv row does: the latent value
is rounded to fp32 and then to bf16 (ties to even both times), the
library's stated decoding (one fp32 product, then the bf16 operand).  The
forward over fp8 kv is the forward of smla_oracle over those rows.
"""
from __future__ import annotations

import numpy as np

from .grouped_oracle import sparse_mla_fwd_grouped
from .smla_oracle import OracleInputError, sparse_mla_fwd

REC_BYTES = 656
SCALE_OFF = 512
ROPE_OFF = 528


def decode_e4m3(codes) -> np.ndarray:
    """fp64 values of e4m3 codes (uint8 array)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, (m / 8.0) * 2.0 ** (1 - 7),
                   (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def decode_kv_records(rec) -> np.ndarray:
    """kv rows [..., 576] (fp64) from fp8 records [..., 656] (uint8)."""
    rec = np.ascontiguousarray(np.asarray(rec, dtype=np.uint8))
    if rec.shape[-1] != REC_BYTES:
        raise OracleInputError(f"fp8 kv records must have {REC_BYTES} bytes")
    lead = rec.shape[:-1]
    flat = rec.reshape(-1, REC_BYTES)
    scales = flat[:, SCALE_OFF:ROPE_OFF].copy().view("<f4").astype(np.float64)   # [n, 4]
    latent = decode_e4m3(flat[:, :SCALE_OFF]) * np.repeat(scales, 128, axis=1)
    rope_bits = flat[:, ROPE_OFF:].copy().view("<u2").astype(np.uint32) << 16
    rope = rope_bits.view(np.float32).astype(np.float64)
    return np.concatenate([latent, rope], axis=1).reshape(*lead, 576)


def round_bf16(x) -> np.ndarray:
    """fp64 values rounded to fp32, then to bf16 (ties to even), as fp64."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    kept = b >> 16
    rem = b & 0xFFFF
    up = (rem > 0x8000) | ((rem == 0x8000) & (kept & 1 == 1))
    r = ((kept + up.astype(np.uint64)) << 16).astype(np.uint32)
    return r.view(np.float32).astype(np.float64)


def kv_rows_bf16(rec) -> np.ndarray:
    """The bf16 kv rows [..., 576] (as fp64) that fp8 records decode to."""
    return round_bf16(decode_kv_records(rec))


def sparse_mla_fwd_fp8(q, kv_rec, idx, sm_scale, d_v=512):
    """out, lse of the forward over decoded fp8 kv records: kv_rec [S_kv, 656]
    with idx [S, K], or [S_kv, G, 656] with idx [S, G, K]."""
    kv = kv_rows_bf16(kv_rec)
    if kv.ndim == 3:
        return sparse_mla_fwd_grouped(q, kv, idx, sm_scale, d_v=d_v)
    return sparse_mla_fwd(q, kv, idx, sm_scale, d_v=d_v)
