"""Per-format dequantization to f32 (oracle; test infrastructure).

Each weight is dequantized from its logical fields with IEEE f32 operations,
round to nearest even, one operation at a time in this order (no fused
multiply-add; NumPy float32 arithmetic rounds after every operation):

  q8_0       32-weight blocks:  w = f32(scale) * f32(q)
  w4a16_g64  64-weight groups:  w = f32(scale) * (f32(q) - f32(zero))
  q4k        256-weight super-blocks of 8 sub-blocks of 32:
                                w = (f32(d) * f32(sc_j)) * f32(q) - f32(dmin) * f32(m_j)
  q6k        256-weight super-blocks of 16 sub-blocks of 16:
                                w = (f32(d) * f32(s_j)) * (f32(q) - 32)
  q4_0       32-weight blocks:  w = f32(d) * (f32(q) - 8),    q in 0..15
  q5_0       32-weight blocks:  w = f32(d) * (f32(q) - 16),   q in 0..31
  q5k        256-weight super-blocks of 8 sub-blocks of 32, q in 0..31:
                                w = (f32(d) * f32(sc_j)) * f32(q) - f32(dmin) * f32(m_j)
  bf16       dense:             w = the bf16 value itself
  i8row      one f32 scale per row:  w = scale_n * f32(q),  q int8

Format names follow the pages: the llmopt README's "packed group-64 W4A16
linear kernels" and its Q4_K and Q5_0 linear parity receipts, the quantized
matvec kernels for Q8_0, Q4_K and Q6_K and the supported tensor types
(q4_0, q5_0, q5_K, bf16) listed in the aot-llm README, and the zynfer PR's
stages M4 (bf16 resident weights, a bf16 x f32 matvec) and M5 (per-row
symmetric int8 weights with fused dequantization).  The pages give no bit
layout or formula; the formulas above are the library's normative
definition (the 32-blocks center their codes on the middle of the code
range, and q5k is q4k with a fifth code bit), and the scale of the group /
sub-block that holds weight k is block index floor(k / block).

For the value ranges of the synthetic workloads every product above is exact
in f32 except i8row's, so the only roundings are the final subtraction of
q4k / q5k (two exact operands, one correctly rounded result) and i8row's one
product of an f32 scale and an integer; the tests check both by recomputing
in f64 and rounding once.
"""
from __future__ import annotations

import numpy as np

from .fp import bf16_to_f32, f16_to_f32

BLOCK = {"q8_0": 32, "w4a16_g64": 64, "q4k": 256, "q6k": 256, "q4_0": 32, "q5_0": 32, "q5k": 256,
         "bf16": 32, "i8row": 32}


def _expand(per_block: np.ndarray, width: int) -> np.ndarray:
    """Repeat each per-block value `width` times along K (block of weight k = k // width)."""
    return np.repeat(per_block, width, axis=-1)


def dequant_q8_0(q, scale) -> np.ndarray:
    s = _expand(f16_to_f32(scale), 32)
    return s * np.asarray(q, dtype=np.int8).astype(np.float32)


def dequant_w4a16_g64(q, scale, zero) -> np.ndarray:
    s = _expand(f16_to_f32(scale), 64)
    z = _expand(f16_to_f32(zero), 64)
    qf = (np.asarray(q, dtype=np.uint8) & 0xF).astype(np.float32)
    return s * (qf - z)


def dequant_q4k(q, sc, m, d, dmin) -> np.ndarray:
    df = _expand(f16_to_f32(d), 256)
    dminf = _expand(f16_to_f32(dmin), 256)
    scf = _expand((np.asarray(sc, dtype=np.uint8) & 0x3F).astype(np.float32), 32)
    mf = _expand((np.asarray(m, dtype=np.uint8) & 0x3F).astype(np.float32), 32)
    qf = (np.asarray(q, dtype=np.uint8) & 0xF).astype(np.float32)
    a = (df * scf) * qf
    b = dminf * mf
    return a - b


def dequant_q6k(q, s, d) -> np.ndarray:
    df = _expand(f16_to_f32(d), 256)
    sf = _expand(np.asarray(s, dtype=np.int8).astype(np.float32), 16)
    qf = (np.asarray(q, dtype=np.uint8) & 0x3F).astype(np.float32)
    return (df * sf) * (qf - np.float32(32.0))


def dequant_q4_0(q, d) -> np.ndarray:
    df = _expand(f16_to_f32(d), 32)
    return df * ((np.asarray(q, dtype=np.uint8) & 0xF).astype(np.float32) - np.float32(8.0))


def dequant_q5_0(q, d) -> np.ndarray:
    df = _expand(f16_to_f32(d), 32)
    return df * ((np.asarray(q, dtype=np.uint8) & 0x1F).astype(np.float32) - np.float32(16.0))


def dequant_q5k(q, sc, m, d, dmin) -> np.ndarray:
    """As q4k, with 5-bit codes."""
    df = _expand(f16_to_f32(d), 256)
    dminf = _expand(f16_to_f32(dmin), 256)
    scf = _expand((np.asarray(sc, dtype=np.uint8) & 0x3F).astype(np.float32), 32)
    mf = _expand((np.asarray(m, dtype=np.uint8) & 0x3F).astype(np.float32), 32)
    qf = (np.asarray(q, dtype=np.uint8) & 0x1F).astype(np.float32)
    return (df * scf) * qf - dminf * mf


def dequant_bf16(q) -> np.ndarray:
    return bf16_to_f32(q)


def dequant_i8row(q, scale) -> np.ndarray:
    s = np.asarray(scale, dtype=np.float32)[..., None]
    return s * np.asarray(q, dtype=np.int8).astype(np.float32)


def dequant(fmt: str, w: dict) -> np.ndarray:
    """Dense f32 [N][K] from the logical arrays of one matrix."""
    if fmt == "q8_0":
        out = dequant_q8_0(w["q"], w["scale"])
    elif fmt == "w4a16_g64":
        out = dequant_w4a16_g64(w["q"], w["scale"], w["zero"])
    elif fmt == "q4k":
        out = dequant_q4k(w["q"], w["sc"], w["m"], w["d"], w["dmin"])
    elif fmt == "q6k":
        out = dequant_q6k(w["q"], w["s"], w["d"])
    elif fmt == "q4_0":
        out = dequant_q4_0(w["q"], w["d"])
    elif fmt == "q5_0":
        out = dequant_q5_0(w["q"], w["d"])
    elif fmt == "q5k":
        out = dequant_q5k(w["q"], w["sc"], w["m"], w["d"], w["dmin"])
    elif fmt == "bf16":
        out = dequant_bf16(w["q"])
    elif fmt == "i8row":
        out = dequant_i8row(w["q"], w["scale"])
    else:
        raise ValueError(f"unknown format {fmt!r}")
    assert out.dtype == np.float32
    return out


def dequant_rows(fmt: str, w: dict, rows) -> np.ndarray:
    """Dequantize only the listed rows (for sampled checks on large matrices)."""
    rows = np.asarray(rows)
    return dequant(fmt, {k: v[rows] for k, v in w.items()})
