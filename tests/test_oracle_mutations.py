"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each test plants one plausible slip into the oracle (by patching it for the
duration of the test) and checks that a hand-worked block or a layout pin
now fails.  The mistakes: sub-block index off by one, sc and m swapped,
d and dmin swapped, the q6 offset dropped, the W4A16 zero's sign flipped,
the nibble order swapped, the two 8-weight halves of a Q6K qh word swapped,
and four slips in the tolerance bound (an L1 norm, a missing square root, the
norm taken over the wrong axis, tau applied twice), the fifth code bit of
Q5_0 / Q5K dropped, the Q4_0 / Q5_0 code offsets swapped, and the per-row
int8 scale applied per column: mutation tests that must fail (pytensor-ml
issue 53, PR 2 item F-60).
"""
import json
import os

import numpy as np

import oracle
from oracle import dequantize as dq
from oracle import layout

from test_oracle_pins import _hand_case, golden, q6k_qh_first_word, tolerance_pin_holds


def _case(cid):
    return next(c for c in golden()["cases"] if c["id"] == cid)


def _y(case):
    w, x = _hand_case(case)
    return oracle.matvec_ref(oracle.dequant(case["fmt"], w), x)[0, 0]


def test_pins_pass_unpatched():
    for c in golden()["cases"]:
        assert _y(c) == c["y"]


def test_subblock_index_off_by_one_is_caught(monkeypatch):
    orig = dq._expand
    monkeypatch.setattr(dq, "_expand", lambda a, width: np.roll(orig(a, width), width, axis=-1))
    bad = [c["id"] for c in golden()["cases"] if _y(c) != c["y"]]
    assert "q4k_e37" in bad and "q6k_e100" in bad


def test_sc_m_swapped_is_caught(monkeypatch):
    orig = dq.dequant_q4k
    monkeypatch.setattr(dq, "dequant_q4k", lambda q, sc, m, d, dmin: orig(q, m, sc, d, dmin))
    assert _y(_case("q4k_ones")) != 3872.0


def test_d_dmin_swapped_is_caught(monkeypatch):
    orig = dq.dequant_q4k
    monkeypatch.setattr(dq, "dequant_q4k", lambda q, sc, m, d, dmin: orig(q, sc, m, dmin, d))
    assert _y(_case("q4k_ones")) != 3872.0


def test_q6_offset_dropped_is_caught(monkeypatch):
    orig = dq.dequant_q6k
    # q - 32 -> q - 0: emulate by adding 32 to q before the oracle subtracts it
    monkeypatch.setattr(dq, "dequant_q6k", lambda q, s, d: orig(np.asarray(q) + 32, s, d))
    assert _y(_case("q6k_e100")) != -1.0


def test_zero_sign_flipped_is_caught(monkeypatch):
    orig = dq.f16_to_f32
    # flip the sign bit of the zero only: patch dequant_w4a16_g64's zero argument
    o = dq.dequant_w4a16_g64
    monkeypatch.setattr(dq, "dequant_w4a16_g64",
                        lambda q, s, z: o(q, s, (np.asarray(z, np.uint16) ^ 0x8000).astype(np.uint16)))
    assert _y(_case("w4a16_ones")) != -8.0
    del orig


def test_nibble_order_swapped_is_caught(monkeypatch):
    def swapped(q):
        q = np.asarray(q, dtype=np.uint8) & 0xF
        return (q[:, 1::2] | (q[:, 0::2] << 4)).astype(np.uint8)
    monkeypatch.setattr(layout, "_nibbles", swapped)
    k = np.arange(64)
    w = {"q": (k % 16).astype(np.uint8)[None], "scale": np.array([[0x3400]], np.uint16),
         "zero": np.array([[0x4800]], np.uint16)}
    buf = oracle.pack_ref("w4a16_g64", w)
    want = {c["id"]: c for c in golden()["packed"]}["w4a16_qs_bytes"]["bytes"]
    assert buf[0] != int(want["0"], 16)


def test_q6k_qh_halves_swapped_is_caught(monkeypatch):
    want = int({c["id"]: c for c in golden()["packed"]}["q6k_qh_word"]["word"], 16)
    assert q6k_qh_first_word() == want

    def swapped(q):
        N, K = q.shape
        hi = ((np.asarray(q, dtype=np.uint8) >> 4) & 3).astype(np.uint32).reshape(N, K // 16, 16)
        w = np.zeros((N, K // 16), dtype=np.uint32)
        for c in range(4):
            for f in range(4):
                k = 8 * (1 - (f >> 1)) + 2 * c + (f & 1)  # the halves exchanged
                w |= hi[:, :, k] << np.uint32(8 * c + 2 * f)
        return w
    monkeypatch.setattr(layout, "_qh_words", swapped)
    assert q6k_qh_first_word() != want


def test_q6k_qh_c_f_roles_swapped_is_caught(monkeypatch):
    want = int({c["id"]: c for c in golden()["packed"]}["q6k_qh_word"]["word"], 16)

    def swapped(q):
        N, K = q.shape
        hi = ((np.asarray(q, dtype=np.uint8) >> 4) & 3).astype(np.uint32).reshape(N, K // 16, 16)
        w = np.zeros((N, K // 16), dtype=np.uint32)
        for c in range(4):
            for f in range(4):
                k = 8 * (f >> 1) + 2 * c + (f & 1)
                w |= hi[:, :, k] << np.uint32(8 * f + 2 * c)  # byte and field index exchanged
        return w
    monkeypatch.setattr(layout, "_qh_words", swapped)
    assert q6k_qh_first_word() != want


def _bound_with(wnorm, xnorm, tau_pow=1):
    def fn(W, x, tau):
        x64 = np.atleast_2d(np.asarray(x, dtype=np.float64))
        W64 = np.asarray(W, dtype=np.float64)
        return (tau ** tau_pow) * xnorm(x64)[:, None] * wnorm(W64)[None, :]
    return fn


_L2_rows = lambda a: np.sqrt(np.sum(a * a, axis=1))  # noqa: E731


def test_tolerance_mutations_are_caught():
    assert tolerance_pin_holds(_bound_with(_L2_rows, _L2_rows))          # the definition itself
    assert tolerance_pin_holds(oracle.tolerance_bound)
    mutants = {
        "L1 norm": _bound_with(lambda a: np.sum(np.abs(a), axis=1), lambda a: np.sum(np.abs(a), axis=1)),
        "no sqrt": _bound_with(lambda a: np.sum(a * a, axis=1), lambda a: np.sum(a * a, axis=1)),
        "W norm over the wrong axis": _bound_with(lambda a: np.sqrt(np.sum(a * a, axis=0)), _L2_rows),
        "x norm over the wrong axis": _bound_with(_L2_rows, lambda a: np.sqrt(np.sum(a * a, axis=0))),
        "tau squared": _bound_with(_L2_rows, _L2_rows, tau_pow=2),
        "max norm": _bound_with(lambda a: np.max(np.abs(a), axis=1), _L2_rows),
    }
    caught = {name: not tolerance_pin_holds(fn) for name, fn in mutants.items()}
    assert all(caught.values()), caught


def test_q5_fifth_bit_dropped_is_caught(monkeypatch):
    o0, ok = dq.dequant_q5_0, dq.dequant_q5k
    monkeypatch.setattr(dq, "dequant_q5_0", lambda q, d: o0(np.asarray(q) & 0xF, d))
    monkeypatch.setattr(dq, "dequant_q5k", lambda q, sc, m, d, dmin: ok(np.asarray(q) & 0xF, sc, m, d, dmin))
    assert _y(_case("q5_0_e21")) != 1.25
    assert _y(_case("q5k_e58")) != 25.5


def test_q4_0_q5_0_offsets_swapped_is_caught(monkeypatch):
    # the Q5_0 offset (16) applied to Q4_0 codes and the Q4_0 offset (8) to Q5_0 codes
    monkeypatch.setattr(dq, "dequant_q4_0", lambda q, d: dq._expand(dq.f16_to_f32(d), 32) * (
        (np.asarray(q) & 0xF).astype(np.float32) - np.float32(16.0)))
    monkeypatch.setattr(dq, "dequant_q5_0", lambda q, d: dq._expand(dq.f16_to_f32(d), 32) * (
        (np.asarray(q) & 0x1F).astype(np.float32) - np.float32(8.0)))
    assert _y(_case("q4_0_ones")) != -8.0
    assert _y(_case("q5_0_ones")) != -4.0


def test_i8row_scale_per_column_is_caught(monkeypatch):
    k = np.arange(32)
    q = np.stack([k - 16, k - 16]).astype(np.int8)
    scale = np.array([0.75, 2.0], np.float32)
    x = np.zeros(32, np.float32)
    x[5] = 1.0

    def pin():
        return np.array_equal(oracle.matvec_ref(oracle.dequant("i8row", {"q": q, "scale": scale}), x),
                              [[-8.25, -22.0]])
    assert pin()
    monkeypatch.setattr(dq, "dequant_i8row", lambda qq, sc: np.resize(np.asarray(sc, np.float32),
                                                                        np.shape(qq)[1])[None, :]
                        * np.asarray(qq, dtype=np.int8).astype(np.float32))
    assert not pin()
