"""Pins of the CPU oracle against values fixed outside it (no GPU).

Each test checks the oracle against something other than itself: library
conversion routines, hand-worked blocks (tests/golden/hand_blocks.json),
exact integer or rational arithmetic, and closed forms.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import dequantize as dq
from oracle import layout
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------- fp decoding

def test_f16_decode_exhaustive_matches_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = oracle.f16_to_f32(bits)
    lib = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan].view(np.uint32), lib[~nan].view(np.uint32))


def test_bf16_decode_exhaustive_matches_torch():
    bits = np.arange(65536, dtype=np.int64)
    mine = oracle.bf16_to_f32(bits.astype(np.uint16))
    t = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    nan = np.isnan(t)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan].view(np.uint32), t[~nan].view(np.uint32))


def test_f16_subnormals_kept():
    assert oracle.f16_to_f64(np.uint16(1))[()] == 2.0 ** -24
    assert oracle.f16_to_f64(np.uint16(0x03FF))[()] == 1023 * 2.0 ** -24
    assert oracle.f16_to_f64(np.uint16(0x8001))[()] == -(2.0 ** -24)


# ---------------------------------------------------------------- hand blocks

def _hand_case(case):
    """Build the logical arrays of one hand-worked block from its formulas."""
    K = case["K"]
    k = np.arange(K)
    fmt = case["fmt"]
    cid = case["id"]
    if fmt == "q8_0":
        w = {"q": (k - 16).astype(np.int8)[None], "scale": np.array([[0x3800]], np.uint16)}
    elif fmt == "w4a16_g64":
        if cid == "w4a16_ones":
            w = {"q": (k % 16).astype(np.uint8)[None], "scale": np.array([[0x3400]], np.uint16),
                 "zero": np.array([[0x4800]], np.uint16)}
        else:
            w = {"q": np.zeros((1, K), np.uint8), "scale": np.array([[0x3400]], np.uint16),
                 "zero": np.array([[0x4680]], np.uint16)}
    elif fmt == "q4k":
        if cid == "q4k_range_edge":
            w = {"q": np.full((1, K), 15, np.uint8), "sc": np.full((1, 8), 63, np.uint8),
                 "m": np.ones((1, 8), np.uint8), "d": np.array([[0x6400]], np.uint16),
                 "dmin": np.array([[0x0001]], np.uint16)}
        else:
            j = np.arange(8)
            w = {"q": (k % 16).astype(np.uint8)[None], "sc": (j + 1).astype(np.uint8)[None],
                 "m": (2 * j).astype(np.uint8)[None], "d": np.array([[0x3800]], np.uint16),
                 "dmin": np.array([[0x3400]], np.uint16)}
    elif fmt == "q6k":
        j = np.arange(16)
        w = {"q": (k % 64).astype(np.uint8)[None], "s": (j - 8).astype(np.int8)[None],
             "d": np.array([[0x3000]], np.uint16)}
    elif fmt == "q4_0":
        w = {"q": (k % 16).astype(np.uint8)[None], "d": np.array([[0x3800]], np.uint16)}
    elif fmt == "q5_0":
        w = {"q": k.astype(np.uint8)[None], "d": np.array([[0x3400]], np.uint16)}
    elif fmt == "q5k":
        j = np.arange(8)
        w = {"q": (k % 32).astype(np.uint8)[None], "sc": (j + 1).astype(np.uint8)[None],
             "m": (2 * j).astype(np.uint8)[None], "d": np.array([[0x3800]], np.uint16),
             "dmin": np.array([[0x3400]], np.uint16)}
    elif fmt == "bf16":
        w = {"q": (0x3F80 + k).astype(np.uint16)[None]}
    else:  # i8row
        w = {"q": (k - 16).astype(np.int8)[None], "scale": np.array([0.75], np.float32)}
    xs = case["x"]
    if xs == "ones":
        x = np.ones(K, np.float32)
    else:
        x = np.zeros(K, np.float32)
        x[int(xs[1:])] = 1.0
    return w, x


@pytest.mark.parametrize("case", golden()["cases"], ids=lambda c: c["id"])
def test_hand_worked_block(case):
    w, x = _hand_case(case)
    W = oracle.dequant(case["fmt"], w)
    y = oracle.matvec_ref(W, x)
    assert y.shape == (1, 1)
    assert y[0, 0] == case["y"]


def test_range_edge_needs_f32_not_f16():
    w, _ = _hand_case(next(c for c in golden()["cases"] if c["id"] == "q4k_range_edge"))
    W = oracle.dequant("q4k", w)
    assert W.dtype == np.float32 and np.all(W == np.float32(967680.0))
    with np.errstate(over="ignore"):
        assert not np.isfinite(np.float16(967680.0))


# ------------------------------------------------------- integer special cases

def _rand_int_x(g, b, K):
    return g.integers(-3, 4, size=(b, K)).astype(np.float32)


def test_q8_0_unit_scale_is_integer_matvec():
    g = np.random.default_rng(7)
    N, K = 5, 96
    q = g.integers(-128, 128, size=(N, K), dtype=np.int8)  # includes -128
    w = {"q": q, "scale": np.full((N, K // 32), 0x3C00, np.uint16)}
    x = _rand_int_x(g, 2, K)
    y = oracle.matvec_ref(oracle.dequant("q8_0", w), x)
    exact = x.astype(np.int64) @ q.astype(np.int64).T
    assert np.array_equal(y, exact.astype(np.float64))


def test_w4a16_unit_scale_integer_zero():
    g = np.random.default_rng(8)
    N, K = 3, 128
    q = g.integers(0, 16, size=(N, K), dtype=np.uint8)
    zint = g.integers(6, 10, size=(N, K // 64))
    w = {"q": q, "scale": np.full((N, K // 64), 0x3C00, np.uint16), "zero": wl.to_f16_bits(zint)}
    x = _rand_int_x(g, 1, K)
    y = oracle.matvec_ref(oracle.dequant("w4a16_g64", w), x)
    wint = q.astype(np.int64) - np.repeat(zint, 64, axis=1)
    assert np.array_equal(y, (x.astype(np.int64) @ wint.T).astype(np.float64))


def test_q4k_unit_d_is_integer_matvec():
    g = np.random.default_rng(9)
    N, K = 3, 512
    w = {"q": g.integers(0, 16, size=(N, K), dtype=np.uint8),
         "sc": g.integers(0, 64, size=(N, K // 32), dtype=np.uint8),
         "m": g.integers(0, 64, size=(N, K // 32), dtype=np.uint8),
         "d": np.full((N, K // 256), 0x3C00, np.uint16),
         "dmin": np.full((N, K // 256), 0x3C00, np.uint16)}
    x = _rand_int_x(g, 2, K)
    y = oracle.matvec_ref(oracle.dequant("q4k", w), x)
    sc = np.repeat(w["sc"].astype(np.int64), 32, axis=1)
    m = np.repeat(w["m"].astype(np.int64), 32, axis=1)
    wint = sc * w["q"].astype(np.int64) - m
    assert np.array_equal(y, (x.astype(np.int64) @ wint.T).astype(np.float64))


def test_q6k_unit_d_is_integer_matvec():
    g = np.random.default_rng(10)
    N, K = 3, 512
    w = {"q": g.integers(0, 64, size=(N, K), dtype=np.uint8),
         "s": g.integers(-64, 64, size=(N, K // 16), dtype=np.int8),
         "d": np.full((N, K // 256), 0x3C00, np.uint16)}
    x = _rand_int_x(g, 2, K)
    y = oracle.matvec_ref(oracle.dequant("q6k", w), x)
    s = np.repeat(w["s"].astype(np.int64), 16, axis=1)
    wint = s * (w["q"].astype(np.int64) - 32)
    assert np.array_equal(y, (x.astype(np.int64) @ wint.T).astype(np.float64))


# ------------------------------------------------- exactness and closed forms

def test_q4_0_q5_0_unit_scale_are_integer_matvecs():
    g = np.random.default_rng(12)
    N, K = 4, 96
    for fmt, bits, off in (("q4_0", 4, 8), ("q5_0", 5, 16)):
        q = g.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
        w = {"q": q, "d": np.full((N, K // 32), 0x3C00, np.uint16)}
        x = _rand_int_x(g, 2, K)
        y = oracle.matvec_ref(oracle.dequant(fmt, w), x)
        assert np.array_equal(y, (x.astype(np.int64) @ (q.astype(np.int64) - off).T).astype(np.float64))


def test_q5k_unit_d_is_integer_matvec():
    g = np.random.default_rng(13)
    N, K = 3, 512
    w = {"q": g.integers(0, 32, size=(N, K), dtype=np.uint8),
         "sc": g.integers(0, 64, size=(N, K // 32), dtype=np.uint8),
         "m": g.integers(0, 64, size=(N, K // 32), dtype=np.uint8),
         "d": np.full((N, K // 256), 0x3C00, np.uint16),
         "dmin": np.full((N, K // 256), 0x3C00, np.uint16)}
    x = _rand_int_x(g, 2, K)
    y = oracle.matvec_ref(oracle.dequant("q5k", w), x)
    wint = np.repeat(w["sc"].astype(np.int64), 32, axis=1) * w["q"].astype(np.int64) - np.repeat(
        w["m"].astype(np.int64), 32, axis=1)
    assert np.array_equal(y, (x.astype(np.int64) @ wint.T).astype(np.float64))


def test_i8row_scale_is_per_row_and_bf16_decodes_like_torch():
    # two rows, scales 0.75 and 2, q = k - 16: x = e5 picks 0.75 * -11 and 2 * -11
    k = np.arange(32)
    w = {"q": np.stack([k - 16, k - 16]).astype(np.int8), "scale": np.array([0.75, 2.0], np.float32)}
    x = np.zeros(32, np.float32)
    x[5] = 1.0
    assert np.array_equal(oracle.matvec_ref(oracle.dequant("i8row", w), x), [[-8.25, -22.0]])
    # unit scale: an integer matvec
    g = np.random.default_rng(14)
    q = g.integers(-128, 128, size=(3, 64), dtype=np.int8)
    xi = _rand_int_x(g, 2, 64)
    y = oracle.matvec_ref(oracle.dequant("i8row", {"q": q, "scale": np.ones(3, np.float32)}), xi)
    assert np.array_equal(y, (xi.astype(np.int64) @ q.astype(np.int64).T).astype(np.float64))
    # bf16 weights are the library conversion's values
    bits = wl.gen_weights("bf16", 4, 64, (91, 0, 0))["q"]
    t = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(oracle.dequant("bf16", {"q": bits}), t)


def test_q4k_single_rounding_matches_f64_difference():
    w = wl.gen_weights("q4k", 64, 1024, (99, 0, 0))
    W = oracle.dequant("q4k", w)
    d = np.repeat(oracle.f16_to_f64(w["d"]), 256, axis=1)
    dm = np.repeat(oracle.f16_to_f64(w["dmin"]), 256, axis=1)
    sc = np.repeat(w["sc"].astype(np.float64), 32, axis=1)
    m = np.repeat(w["m"].astype(np.float64), 32, axis=1)
    exact = d * sc * w["q"] - dm * m          # exact in f64 for these ranges
    assert np.array_equal(W, exact.astype(np.float32))


@pytest.mark.parametrize("fmt", wl.FORMATS)
def test_dequant_exact_rational_on_workload_ranges(fmt):
    """For the workload value ranges no product rounds (q4k: only the final subtraction)."""
    K = 256
    w = wl.gen_weights(fmt, 2, K, (98, 0, wl.FORMATS.index(fmt)))
    W = oracle.dequant(fmt, w)
    F = lambda b: Fraction(float(oracle.f16_to_f64(np.uint16(b))[()]))  # noqa: E731
    for n in range(2):
        for kk in range(0, K, 7):
            if fmt == "q8_0":
                e = F(w["scale"][n, kk // 32]) * int(w["q"][n, kk])
            elif fmt == "w4a16_g64":
                e = F(w["scale"][n, kk // 64]) * (int(w["q"][n, kk]) - F(w["zero"][n, kk // 64]))
            elif fmt == "q4k":
                e = (F(w["d"][n, kk // 256]) * int(w["sc"][n, kk // 32]) * int(w["q"][n, kk])
                     - F(w["dmin"][n, kk // 256]) * int(w["m"][n, kk // 32]))
            elif fmt == "q6k":
                e = F(w["d"][n, kk // 256]) * int(w["s"][n, kk // 16]) * (int(w["q"][n, kk]) - 32)
            elif fmt == "q4_0":
                e = F(w["d"][n, kk // 32]) * (int(w["q"][n, kk]) - 8)
            elif fmt == "q5_0":
                e = F(w["d"][n, kk // 32]) * (int(w["q"][n, kk]) - 16)
            elif fmt == "q5k":
                e = (F(w["d"][n, kk // 256]) * int(w["sc"][n, kk // 32]) * int(w["q"][n, kk])
                     - F(w["dmin"][n, kk // 256]) * int(w["m"][n, kk // 32]))
            elif fmt == "bf16":
                e = Fraction(float(oracle.bf16_to_f64(np.uint16(w["q"][n, kk]))[()]))
            else:  # i8row: one correctly rounded f32 product
                e = Fraction(float(w["scale"][n])) * int(w["q"][n, kk])
            if fmt in ("q4k", "q5k", "i8row"):
                assert float(W[n, kk]) == float(np.float32(float(e)))  # f64 holds e exactly; one rounding
            else:
                assert Fraction(float(W[n, kk])) == e


@pytest.mark.parametrize("fmt", wl.FORMATS)
def test_f64_accumulation_against_fractions(fmt):
    """Brute force: exact rational sums equal the f64 reference to ~1 ulp."""
    K = wl.BLOCK[fmt] * 2
    for N in (1, 3, 4):
        w = wl.gen_weights(fmt, N, K, (97, N, wl.FORMATS.index(fmt)))
        x = wl.gen_x(K, 2, "f32", (97, N, wl.FORMATS.index(fmt)))
        W = oracle.dequant(fmt, w)
        y = oracle.matvec_ref(W, x)
        for b in range(2):
            for n in range(N):
                exact = sum(Fraction(float(W[n, k])) * Fraction(float(x[b, k])) for k in range(K))
                scale = sum(abs(Fraction(float(W[n, k])) * Fraction(float(x[b, k]))) for k in range(K))
                assert abs(Fraction(y[b, n]) - exact) <= scale * Fraction(K, 2 ** 52)


def test_closed_forms():
    K = 256
    # q6k: q = 32 everywhere gives w = 0 and y = 0 exactly
    w = wl.gen_weights("q6k", 3, K, (96, 0, 0))
    w["q"][:] = 32
    assert np.all(oracle.dequant("q6k", w) == 0)
    # q4k: q = 0 gives w = -dmin * m on every weight of the sub-block
    w = wl.gen_weights("q4k", 3, K, (96, 0, 1))
    w["q"][:] = 0
    W = oracle.dequant("q4k", w)
    want = -(oracle.f16_to_f64(w["dmin"])[:, :, None] * w["m"].reshape(3, 1, 8).astype(np.float64))
    assert np.array_equal(W.reshape(3, 8, 32), np.broadcast_to(want.reshape(3, 8, 1), (3, 8, 32)).astype(np.float32))
    # x = ones gives the exact row sums (f64 sum of exact f32 weights, fsum as the library routine)
    import math
    x = np.ones((1, K), np.float32)
    y = oracle.matvec_ref(W, x)
    for n in range(3):
        assert y[0, n] == pytest.approx(math.fsum(map(float, W[n])), rel=1e-15, abs=1e-300)


def test_gemm_reduces_to_torch_matmul():
    g = np.random.default_rng(11)
    w = wl.gen_weights("w4a16_g64", 40, 128, (95, 0, 0))
    W = oracle.dequant("w4a16_g64", w)
    Xb = wl.gen_x(128, 5, "bf16", (95, 0, 0))
    X = oracle.bf16_to_f32(Xb)
    Y = oracle.gemm_ref(W, X)
    T = (torch.from_numpy(X).double() @ torch.from_numpy(W).double().T).numpy()
    assert np.allclose(Y, T, rtol=1e-12, atol=1e-12)
    del g


def test_tolerance_check_flags_errors():
    w = wl.gen_weights("q4k", 8, 256, (94, 0, 0))
    W = oracle.dequant("q4k", w)
    x = wl.gen_x(256, 1, "f32", (94, 0, 0))
    y = oracle.matvec_ref(W, x)
    bound = oracle.tolerance_bound(W, x, 1e-3)
    assert oracle.check_within(y, y, bound)["ok"]
    bad = y.copy()
    bad[0, 3] += 2 * bound[0, 3]
    r = oracle.check_within(bad, y, bound)
    assert not r["ok"] and r["max_ratio"] > 1.5


def tolerance_pin_holds(bound_fn) -> bool:
    """The hand-worked tolerance case (tests/golden/hand_blocks.json, "tolerance"):
    bound_fn(W, x, tau) must give exactly the printed bounds."""
    c = golden()["tolerance"][0]
    W = np.array(c["W"], np.float32)
    x = np.array(c["x"], np.float32)
    try:
        got = np.asarray(bound_fn(W, x, c["tau"]), dtype=np.float64)
    except Exception:
        return False
    want = np.array(c["bound"], np.float64)
    return got.shape == want.shape and bool(np.array_equal(got, want))


def test_tolerance_bound_hand_worked():
    assert tolerance_pin_holds(oracle.tolerance_bound)
    # a single vector is broadcast as one batch row
    c = golden()["tolerance"][0]
    b = oracle.tolerance_bound(np.array(c["W"], np.float32), np.array(c["x"][0], np.float32), 1e-3)
    assert b.shape == (1, 2) and b[0, 0] == pytest.approx(15e-3) and b[0, 1] == pytest.approx(39e-3)


def test_check_within_hand_worked():
    ref = np.array([[1.0, -2.0]])
    bound = np.array([[0.5, 0.25]])
    assert oracle.check_within(np.array([[1.5, -2.25]]), ref, bound)["ok"]        # exactly on the bound
    assert not oracle.check_within(np.array([[1.5000001, -2.0]]), ref, bound)["ok"]
    assert not oracle.check_within(np.array([[np.nan, -2.0]]), ref, bound)["ok"]
    r = oracle.check_within(np.array([[1.25, -2.0]]), ref, bound)
    assert r["ok"] and r["max_ratio"] == 0.5 and r["max_abs"] == 0.25 and r["n_exact_f32"] == 1


# ---------------------------------------------------------------- layout pins

def test_packed_bytes_hand_worked():
    G = {c["id"]: c for c in golden()["packed"]}
    k = np.arange(64)
    w = {"q": (k % 16).astype(np.uint8)[None], "scale": np.array([[0x3400]], np.uint16),
         "zero": np.array([[0x4800]], np.uint16)}
    buf = oracle.pack_ref("w4a16_g64", w)
    for pos, val in G["w4a16_qs_bytes"]["bytes"].items():
        assert buf[int(pos)] == int(val, 16)
    off, _ = layout.plane_offsets("w4a16_g64", 1, 64)["sz"]
    assert buf[off:off + 4].view(np.uint32)[0] == int(G["w4a16_sz_word"]["word"], 16)

    j = np.arange(8)
    w = {"q": np.zeros((1, 256), np.uint8), "sc": (j + 1).astype(np.uint8)[None],
         "m": (2 * j).astype(np.uint8)[None], "d": np.array([[0x3800]], np.uint16),
         "dmin": np.array([[0x3400]], np.uint16)}
    buf = oracle.pack_ref("q4k", w)
    off, nb = layout.plane_offsets("q4k", 1, 256)["meta"]
    assert buf[off:off + nb].tobytes().hex() == G["q4k_meta_record"]["hex"]

    assert q6k_qh_first_word() == int(G["q6k_qh_word"]["word"], 16)


Q6K_QH_PATTERN = (0, 1, 2, 3, 3, 2, 1, 0, 1, 3, 0, 2, 2, 0, 3, 1)  # high bits h(k), k = 0..15


def q6k_qh_first_word() -> int:
    """First qh word the oracle packs for q = 16 h(k) + (k mod 16), the golden pattern."""
    k = np.arange(256)
    h = np.array(Q6K_QH_PATTERN * 16)
    w = {"q": (16 * h + (k % 16)).astype(np.uint8)[None], "s": np.zeros((1, 16), np.int8),
         "d": np.array([[0]], np.uint16)}
    buf = oracle.pack_ref("q6k", w)
    off, _ = layout.plane_offsets("q6k", 1, 256)["qh"]
    return int(buf[off:off + 4].view(np.uint32)[0])


def test_q5_qh_word_hand_worked():
    G = {c["id"]: c for c in golden()["packed"]}
    k = np.arange(32)
    h = np.isin(k, [3, 8, 21, 30]).astype(np.uint8)
    w = {"q": (16 * h + (k % 16)).astype(np.uint8)[None], "d": np.array([[0x3C00]], np.uint16)}
    buf = oracle.pack_ref("q5_0", w)
    off, _ = layout.plane_offsets("q5_0", 1, 32)["qh"]
    assert buf[off:off + 4].view(np.uint32)[0] == int(G["q5_qh_word"]["word"], 16)


@pytest.mark.parametrize("fmt", wl.FORMATS)
def test_pack_unpack_round_trip(fmt):
    N, K = 7, wl.BLOCK[fmt] * 3
    w = wl.gen_weights(fmt, N, K, (93, 0, wl.FORMATS.index(fmt)))
    buf = oracle.pack_ref(fmt, w)
    assert buf.size == oracle.packed_bytes_ref(fmt, N, K) and buf.size % 256 == 0
    back = oracle.unpack_ref(fmt, N, K, buf)
    assert set(back) == set(w)
    for name in w:
        assert np.array_equal(back[name], w[name]), name


def test_packed_sizes_match_bits_per_weight():
    # plane bytes (without padding) per weight: 8.5, 4.5, 4.5, 6.5625 bits
    for fmt, bits in (("q8_0", 8.5), ("w4a16_g64", 4.5), ("q4k", 4.5), ("q6k", 6.5625), ("q4_0", 4.5),
                      ("q5_0", 5.5), ("q5k", 5.5), ("bf16", 16.0), ("i8row", 8.0 + 32 / 4096)):
        N, K = 256, 4096
        raw = sum(nb for _, nb in layout._planes(fmt, N, K))
        assert raw * 8 == bits * N * K


# ---------------------------------------------------------------- generators

def test_generators_deterministic_and_in_range():
    for fmt in wl.FORMATS:
        a = wl.gen_weights(fmt, 4, 512, (92, 1, 2))
        b = wl.gen_weights(fmt, 4, 512, (92, 1, 2))
        for k in a:
            assert np.array_equal(a[k], b[k])
    w = wl.gen_weights("q8_0", 64, 512, (92, 0, 0))
    assert w["q"].min() >= -127 and w["q"].max() <= 127
    w = wl.gen_weights("w4a16_g64", 64, 512, (92, 0, 1))
    z = oracle.f16_to_f32(w["zero"])
    assert w["q"].max() <= 15 and z.min() >= 6.0 and z.max() <= 9.0
    w = wl.gen_weights("q4k", 64, 512, (92, 0, 2))
    assert w["sc"].max() <= 63 and w["m"].max() <= 63 and w["q"].max() <= 15
    w = wl.gen_weights("q6k", 64, 512, (92, 0, 3))
    assert w["q"].max() <= 63 and w["s"].min() >= -64 and w["s"].max() <= 63
    assert wl.gen_weights("q4_0", 64, 512, (92, 0, 4))["q"].max() == 15
    assert wl.gen_weights("q5_0", 64, 512, (92, 0, 5))["q"].max() == 31
    w = wl.gen_weights("q5k", 64, 512, (92, 0, 6))
    assert w["q"].max() == 31 and w["sc"].max() <= 63 and w["m"].max() <= 63
    w = wl.gen_weights("i8row", 64, 512, (92, 0, 7))
    assert w["q"].min() >= -127 and w["scale"].dtype == np.float32 and w["scale"].shape == (64,)
    assert np.all(np.isfinite(oracle.dequant("bf16", wl.gen_weights("bf16", 64, 512, (92, 0, 8)))))
    x1 = wl.gen_x(512, 2, "f32", (92, 0, 0))
    x2 = wl.gen_x(512, 2, "f32", (92, 0, 0))
    assert np.array_equal(x1, x2)


def test_workload_tables():
    c5 = wl.c5_sweep(1)
    assert len(c5["mats"]) == 155
    total = sum(wl.bytes_per_weight(f) * N * K for _, f, N, K, _ in c5["mats"])
    assert total == 667152384
