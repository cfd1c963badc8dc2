"""Activations quantized to 8-bit blocks, and the matvec over them (oracle;
test infrastructure).

The pages' CPU decode path quantizes the f32 activation vector once per
matmul to 8-bit blocks and computes every output row as integer dot products
scaled back to f32 (aot-llm README, "How it works", CPU paragraph; its error
against an f64 reference is about 1e-3, where the f32-activation path is
about 1e-6: Metal backend notes).  The pages do not spell out the rounding;
the library's definition, per vector and per block of 32 activations
x[32j .. 32j + 31] (f32):

    amax = max_k |x_k|
    d    = amax / 127           (f32 division, round to nearest even)
    id   = 127 / amax           (f32 division)
    q_k  = rint(x_k * id)       (f32 product, then round half to even to an
                                 integer), clamped to [-127, 127]

except that a block with amax < 2^-120 (all zero, or so small that 127 / amax
would overflow f32 near amax = 3.7e-37) takes d = id = 0 and all codes 0: it
quantizes to exact zeros.  Inputs must be finite.

and the quantized activation is x^_k = d * q_k, exactly (an f64 product).
Every step is one IEEE f32 operation, so the codes and scales are unique bit
for bit and the GPU quantizer is compared with these exactly.  The product
over the quantized vector is then the plain f64 matvec of the dequantized
weights against x^.
"""
from __future__ import annotations

import numpy as np


def quantize_q8x(x) -> tuple[np.ndarray, np.ndarray]:
    """x f32 [b][K] (K a multiple of 32) -> (q int8 [b][K], d f32 [b][K/32])."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float32))
    b, K = x.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    blocks = x.reshape(b, K // 32, 32)
    amax = np.max(np.abs(blocks), axis=2)                      # exact
    live = amax >= np.float32(2.0 ** -120)
    with np.errstate(divide="ignore", over="ignore"):
        d = np.where(live, amax / np.float32(127.0), np.float32(0.0)).astype(np.float32)    # one f32 division
        id_ = np.where(live, np.float32(127.0) / amax, np.float32(0.0)).astype(np.float32)  # one f32 division
    prod = (blocks * id_[:, :, None]).astype(np.float32)       # one f32 product
    q = np.clip(np.rint(prod), -127, 127).astype(np.int8)      # round half to even
    return q.reshape(b, K), d


def dequant_q8x(q, d) -> np.ndarray:
    """x^ = d * q in f64 (exact)."""
    q = np.atleast_2d(np.asarray(q, dtype=np.int8)).astype(np.float64)
    b, K = q.shape
    return q * np.repeat(np.asarray(d, dtype=np.float32).astype(np.float64), 32, axis=1).reshape(b, K)


def q8x_record_bytes(K: int) -> int:
    """Bytes of one quantized vector in the library's buffer: K codes, then K/32
    f32 scales, the record rounded up to 16 bytes."""
    return (K + K // 8 + 15) // 16 * 16


def pack_q8x(q, d) -> np.ndarray:
    """The library's buffer layout of quantized activations (vector b at b * record)."""
    q = np.atleast_2d(np.asarray(q, dtype=np.int8))
    b, K = q.shape
    rec = q8x_record_bytes(K)
    out = np.zeros(b * rec, dtype=np.uint8)
    for i in range(b):
        out[i * rec:i * rec + K] = q[i].view(np.uint8)
        out[i * rec + K:i * rec + K + K // 8] = np.asarray(d[i], dtype=np.float32).view(np.uint8)
    return out
