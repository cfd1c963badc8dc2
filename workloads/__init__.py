"""Seeded synthetic inputs for block-quantized matvec and GEMM workloads.

This module only *draws* inputs: small integers for the quantized fields,
fp16/bf16 bit patterns for scales and activations, and the shape tables of
the workloads.  It contains none of the dequantization or product arithmetic:
both the CPU oracle and the HIP path receive the arrays it returns.

Logical (unpacked) arrays, row-major, one entry per weight or per block:

  q8_0       q int8 [N][K] in [-127, 127]; scale f16 [N][K/32]
  w4a16_g64  q uint8 [N][K] in [0, 15]; scale f16 [N][K/64]; zero f16 [N][K/64]
  q4k        q uint8 [N][K] in [0, 15]; sc, m uint8 [N][K/32] in [0, 63];
             d, dmin f16 [N][K/256]
  q6k        q uint8 [N][K] in [0, 63]; s int8 [N][K/16] in [-64, 63];
             d f16 [N][K/256]
  q4_0       q uint8 [N][K] in [0, 15]; d f16 [N][K/32]
  q5_0       q uint8 [N][K] in [0, 31]; d f16 [N][K/32]
  q5k        q uint8 [N][K] in [0, 31]; sc, m uint8 [N][K/32] in [0, 63];
             d, dmin f16 [N][K/256]
  bf16       q uint16 [N][K]: bf16 bit patterns of the weights themselves
  i8row      q int8 [N][K] in [-127, 127]; scale f32 [N] (one per row)

The parameter distributions of the last five (formats the pages name but
give no workload for) follow the nearest given ones: 32-blocks like Q8_0's
scale, Q5K like Q4K, bf16 weights 0.02 N(0,1), per-row int8 scales like
Q8_0's but in f32.

f16/bf16 arrays are returned as their uint16 bit patterns.  Scale-like values
are drawn in float64 and rounded once to fp16 (round to nearest even),
keeping subnormals and zeros.

The shapes are those of a 1.1B-parameter Llama-style decoder (dim 2048,
MLP 5632, 22 layers, 32 query / 4 KV heads of 64, vocab 32000) as printed in
the aot-llm README's compile transcript, and of a 0.6B decoder MLP (1024 /
3072, vocab 151936).  No trained weights are involved: every value is random.
"""
from __future__ import annotations

import numpy as np

FORMATS = ("q8_0", "w4a16_g64", "q4k", "q6k", "q4_0", "q5_0", "q5k", "bf16", "i8row")

# K must be a multiple of this for each format (its block, or the kernels'
# 32-weight unit for the formats without blocks)
BLOCK = {"q8_0": 32, "w4a16_g64": 64, "q4k": 256, "q6k": 256, "q4_0": 32, "q5_0": 32, "q5k": 256,
         "bf16": 32, "i8row": 32}

# The field names of each format's logical arrays, in the order the C ABI's
# qmv_logical.aux[] takes them (q is separate).
AUX_FIELDS = {
    "q8_0": ("scale",),
    "w4a16_g64": ("scale", "zero"),
    "q4k": ("sc", "m", "d", "dmin"),
    "q6k": ("s", "d"),
    "q4_0": ("d",),
    "q5_0": ("d",),
    "q5k": ("sc", "m", "d", "dmin"),
    "bf16": (),
    "i8row": ("scale",),
}


def rng_for(*key: int) -> np.random.Generator:
    """PCG64 generator for a workload key (config, layer, matrix, stream)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([2026, *key])))


def to_f16_bits(a: np.ndarray) -> np.ndarray:
    """Round float64 values once to fp16 (RNE) and return the bit patterns."""
    return np.asarray(a, dtype=np.float64).astype(np.float16).view(np.uint16)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (via f32, RNE on the dropped 16 bits)."""
    f = np.asarray(a, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def gen_weights(fmt: str, N: int, K: int, key: tuple) -> dict:
    """Logical arrays of one N x K matrix in format `fmt`, seeded by `key`.

    Draw order: q first, then the aux arrays in AUX_FIELDS order.
    """
    if fmt not in BLOCK:
        raise ValueError(f"unknown format {fmt!r}")
    if K % BLOCK[fmt]:
        raise ValueError(f"K={K} is not a multiple of {BLOCK[fmt]} for {fmt}")
    g = rng_for(*key, 0)
    out = {}
    if fmt == "q8_0":
        out["q"] = g.integers(-127, 128, size=(N, K), dtype=np.int8)
        out["scale"] = to_f16_bits(0.01 * np.abs(g.standard_normal((N, K // 32))) + 1e-4)
    elif fmt == "w4a16_g64":
        out["q"] = g.integers(0, 16, size=(N, K), dtype=np.uint8)
        out["scale"] = to_f16_bits(0.02 * np.abs(g.standard_normal((N, K // 64))) + 1e-4)
        out["zero"] = to_f16_bits(g.uniform(6.0, 9.0, size=(N, K // 64)))
    elif fmt == "q4k":
        out["q"] = g.integers(0, 16, size=(N, K), dtype=np.uint8)
        out["sc"] = g.integers(0, 64, size=(N, K // 32), dtype=np.uint8)
        out["m"] = g.integers(0, 64, size=(N, K // 32), dtype=np.uint8)
        out["d"] = to_f16_bits(1e-3 * np.abs(g.standard_normal((N, K // 256))))
        out["dmin"] = to_f16_bits(1e-3 * np.abs(g.standard_normal((N, K // 256))))
    elif fmt == "q6k":
        out["q"] = g.integers(0, 64, size=(N, K), dtype=np.uint8)
        out["s"] = g.integers(-64, 64, size=(N, K // 16), dtype=np.int8)
        out["d"] = to_f16_bits(1e-3 * np.abs(g.standard_normal((N, K // 256))))
    elif fmt in ("q4_0", "q5_0"):
        out["q"] = g.integers(0, 16 if fmt == "q4_0" else 32, size=(N, K), dtype=np.uint8)
        out["d"] = to_f16_bits(0.01 * np.abs(g.standard_normal((N, K // 32))) + 1e-4)
    elif fmt == "q5k":
        out["q"] = g.integers(0, 32, size=(N, K), dtype=np.uint8)
        out["sc"] = g.integers(0, 64, size=(N, K // 32), dtype=np.uint8)
        out["m"] = g.integers(0, 64, size=(N, K // 32), dtype=np.uint8)
        out["d"] = to_f16_bits(1e-3 * np.abs(g.standard_normal((N, K // 256))))
        out["dmin"] = to_f16_bits(1e-3 * np.abs(g.standard_normal((N, K // 256))))
    elif fmt == "bf16":
        out["q"] = to_bf16_bits(0.02 * g.standard_normal((N, K)))
    else:  # i8row
        out["q"] = g.integers(-127, 128, size=(N, K), dtype=np.int8)
        out["scale"] = (0.01 * np.abs(g.standard_normal(N)) + 1e-4).astype(np.float32)
    return out


def gen_x(K: int, batch: int, dtype: str, key: tuple) -> np.ndarray:
    """Activations [batch][K] drawn N(0,1).

    dtype "f32" -> float32 values; "f16" / "bf16" -> uint16 bit patterns.
    Drawn from a stream of their own (key + (1,)), independent of the weights.
    """
    v = rng_for(*key, 1).standard_normal((batch, K))
    if dtype == "f32":
        return v.astype(np.float32)
    if dtype == "f16":
        return to_f16_bits(v)
    if dtype == "bf16":
        return to_bf16_bits(v)
    raise ValueError(f"unknown activation dtype {dtype!r}")


# --------------------------------------------------------------------------
# Workload tables.  Each matrix: (name, fmt, N, K, key).  Keys are
# (config id, layer, matrix index); layer 1000 marks matrices outside layers.

LLAMA_1B1 = dict(dim=2048, mlp=5632, layers=22, heads=32, kv_heads=4, head_dim=64, vocab=32000)


def c1_q8_0():
    """Q8_0 512 x 512 matvec, batch 1, f32 x."""
    return dict(name="q8_0 512x512 b1", x_dtype="f32", batch=1,
                mats=[("w", "q8_0", 512, 512, (1, 0, 0))])


def c2_w4a16_mlp():
    """Group-64 W4A16 decode matvecs on 1.1B-decoder MLP shapes, batch 1, f16 x."""
    d, f = LLAMA_1B1["dim"], LLAMA_1B1["mlp"]
    return dict(name="w4a16_g64 1.1B MLP b1", x_dtype="f16", batch=1,
                mats=[("gate", "w4a16_g64", f, d, (2, 0, 4)),
                      ("up", "w4a16_g64", f, d, (2, 0, 5)),
                      ("down", "w4a16_g64", d, f, (2, 0, 6))])


def c3_q4k_0b6():
    """Q4K matvecs on a 0.6B decoder's MLP and its 151936-row vocab head, f32 x."""
    return dict(name="q4k 0.6B MLP+head b1", x_dtype="f32", batch=1,
                mats=[("up", "q4k", 3072, 1024, (3, 0, 5)),
                      ("down", "q4k", 1024, 3072, (3, 0, 6)),
                      ("head", "q4k", 151936, 1024, (3, 1000, 7))])


def c4_gemm(M: int):
    """W4A16 prefill GEMM: X [M][2048] bf16 times W^T, W 5632 x 2048."""
    return dict(name=f"w4a16_g64 GEMM M={M}", x_dtype="bf16", batch=M,
                mats=[("gate", "w4a16_g64", 5632, 2048, (4, 0, 4))])


# matrix index follows the decode order q, k, v, o, gate, up, down; head = 7
C5_LAYER = (("q", "q4k", 2048, 2048), ("k", "q4k", 256, 2048), ("v", "q6k", 256, 2048),
            ("o", "q4k", 2048, 2048), ("gate", "q4k", 5632, 2048), ("up", "q4k", 5632, 2048),
            ("down", "q6k", 2048, 5632))


def c5_sweep(batch: int, layers: int = 22):
    """Every matvec of one decode token of the 1.1B decoder, in forward order."""
    mats = []
    for L in range(layers):
        for i, (nm, fmt, N, K) in enumerate(C5_LAYER):
            mats.append((f"l{L}.{nm}", fmt, N, K, (5, L, i)))
    mats.append(("head", "q6k", LLAMA_1B1["vocab"], LLAMA_1B1["dim"], (5, 1000, 7)))
    return dict(name=f"1.1B decode sweep b{batch}", x_dtype="f32", batch=batch, mats=mats)


def bytes_per_weight(fmt: str, K: int | None = None) -> float:
    """Algorithmic bytes per weight (quantized fields + scales/mins); i8row's
    per-row scale needs the row length K."""
    if fmt == "i8row":
        return 1.0 + 4.0 / K
    return {"q8_0": 34 / 32, "w4a16_g64": 36 / 64, "q4k": 144 / 256, "q6k": 210 / 256,
            "q4_0": 18 / 32, "q5_0": 22 / 32, "q5k": 176 / 256, "bf16": 2.0}[fmt]
