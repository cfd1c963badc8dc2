"""Pins of the 8-bit activation quantizer of the integer-dot variant (no GPU).

Hand-worked blocks (tests/golden/hand_blocks.json, "q8act"): a ramp whose
scaled values are exact in f32 (so every code follows by hand), ties that
separate round-half-to-even from round-half-away, and the all-zero block;
plus the per-block (not per-vector) scale, the exactness of d * q in f64,
the error bound of the quantization, and planted mistakes.
"""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.json")


def _cases():
    return {c["id"]: c for c in json.load(open(GOLDEN))["q8act"]}


def _x(cid):
    k = np.arange(32)
    if cid == "q8x_ramp":
        return (0.25 * (k - 16)).astype(np.float32)[None]
    if cid == "q8x_halfway":
        x = np.zeros((1, 32), np.float32)
        x[0, :6] = [127, 2.5, 3.5, -2.5, -0.5, 0.5]
        return x
    return np.zeros((1, 32), np.float32)


def pins_hold(quant) -> bool:
    for cid, c in _cases().items():
        q, d = quant(_x(cid))
        if list(np.asarray(q)[0].astype(int)) != c["q"]:
            return False
        if int(np.asarray(d, np.float32).view(np.uint32)[0, 0]) != int(c["d_bits"], 16):
            return False
    return True


def test_hand_worked_blocks():
    assert pins_hold(oracle.quantize_q8x)


def test_scale_is_per_block_and_dequant_exact():
    x = np.concatenate([_x("q8x_ramp"), _x("q8x_halfway")], axis=1)  # two blocks
    q, d = oracle.quantize_q8x(x)
    assert d.shape == (1, 2) and d[0, 0] == np.float32(4) / np.float32(127) and d[0, 1] == 1.0
    xh = oracle.dequant_q8x(q, d)
    assert np.array_equal(xh[0, 32:38], [127, 2, 4, -2, 0, 0])
    assert xh[0, 1] == float(np.float32(4) / np.float32(127)) * -119  # exact f64 product


def test_quantization_error_bound():
    # |x - x^| <= d / 2 (one rounding of x * id, plus the f32 rounding of id and d)
    x = np.random.default_rng(5).normal(0, 1, (4, 2048)).astype(np.float32)
    q, d = oracle.quantize_q8x(x)
    err = np.abs(x.astype(np.float64) - oracle.dequant_q8x(q, d))
    half = np.repeat(d.astype(np.float64), 32, axis=1) * (0.5 + 1e-5)
    assert np.all(err <= half) and np.all(np.abs(q) <= 127)


def test_buffer_layout():
    x = np.random.default_rng(6).normal(0, 1, (3, 96)).astype(np.float32)
    q, d = oracle.quantize_q8x(x)
    buf = oracle.pack_q8x(q, d)
    rec = oracle.q8x_record_bytes(96)
    assert rec == 112 and buf.size == 3 * rec
    assert np.array_equal(buf[rec:rec + 96].view(np.int8), q[1])
    assert np.array_equal(buf[rec + 96:rec + 108].view(np.float32), d[1])


def test_mutations_are_caught():
    def half_away(x):
        q, d = oracle.quantize_q8x(x)
        x = np.atleast_2d(np.asarray(x, np.float32))
        amax = np.max(np.abs(x.reshape(x.shape[0], -1, 32)), axis=2)
        id_ = np.where(amax > 0, np.float32(127) / amax, 0).astype(np.float32)
        p = (x.reshape(x.shape[0], -1, 32) * id_[:, :, None]).astype(np.float32)
        return np.clip(np.sign(p) * np.floor(np.abs(p) + 0.5), -127, 127).astype(np.int8).reshape(x.shape), d

    def over_128(x):
        q, d = oracle.quantize_q8x(x)
        return q, (np.asarray(d) * np.float32(127) / np.float32(128)).astype(np.float32)

    def per_vector(x):
        x = np.atleast_2d(np.asarray(x, np.float32))
        amax = np.max(np.abs(x), axis=1, keepdims=True)
        d = np.repeat((amax / np.float32(127)).astype(np.float32), x.shape[1] // 32, axis=1)
        id_ = np.where(amax > 0, np.float32(127) / amax, 0).astype(np.float32)
        return np.clip(np.rint((x * id_).astype(np.float32)), -127, 127).astype(np.int8), d

    for m in (half_away, over_128):
        assert not pins_hold(m), m.__name__
    two = np.concatenate([_x("q8x_ramp"), _x("q8x_halfway")], axis=1)
    assert not np.array_equal(per_vector(two)[1], oracle.quantize_q8x(two)[1])


def test_tiny_blocks_quantize_to_zero():
    # 127 / amax overflows f32 below amax ~ 3.7e-37: such a block (threshold
    # 2^-120) quantizes to exact zeros; at the threshold itself id = 127 * 2^120
    # is exact and a half-way product rounds to even.
    x = np.zeros((1, 64), np.float32)
    x[0, 0], x[0, 1] = 1e-37, -5e-38
    x[0, 32], x[0, 33] = 2.0 ** -120, -(2.0 ** -121)
    q, d = oracle.quantize_q8x(x)
    assert not np.any(q[0, :32]) and d[0, 0] == 0.0
    assert q[0, 32] == 127 and q[0, 33] == -64 and not np.any(q[0, 34:])
    assert d[0, 1] == np.float32(2.0 ** -120) / np.float32(127)
    assert np.all(np.isfinite(oracle.dequant_q8x(q, d)))
