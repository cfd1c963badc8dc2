"""Host-side checks of libqmv (no GPU): the library loads, exports every entry
point its header declares, sizes packed buffers like the reference layout,
and rejects bad arguments before touching a device."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmv.h")


@pytest.fixture(scope="module")
def q():
    import gemm_dequant_matvec_amd as mod
    return mod


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qmv_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(
        ["qmv_abi_version", "qmv_status_string", "qmv_last_error", "qmv_packed_bytes",
         "qmv_pack", "qmv_matvec", "qmv_matvec_ex", "qmv_matvec_swiglu", "qmv_matvec_grouped", "qmv_gemm",
         "qmv_dequant", "qmv_quantize_x", "qmv_q8x_bytes"])


def test_library_exports_every_declared_symbol(q):
    lib = ctypes.CDLL(q.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(q.EXPORTS) == set(declared_functions())


def test_abi_and_status_strings(q):
    assert q.abi_version() == (3, 1)
    for st in range(0, -10, -1):
        assert q._lib.qmv_status_string(st).decode() not in ("", "unknown status")
    assert q._lib.qmv_status_string(-99).decode() == "unknown status"


@pytest.mark.parametrize("fmt", wl.FORMATS)
@pytest.mark.parametrize("N,mult,batch", [(1, 1, 1), (7, 3, 2), (300, 8, 1), (5632, 8, 3)])
def test_packed_bytes_matches_reference_layout(q, fmt, N, mult, batch):
    K = wl.BLOCK[fmt] * mult
    assert q.packed_bytes(fmt, N, K, batch) == oracle.packed_bytes_ref(fmt, N, K, batch)


def test_packed_bytes_errors(q):
    out = ctypes.c_size_t(0)
    assert q.raw_call("qmv_packed_bytes", 10, 4, 32, 1, ctypes.byref(out)) == -2
    assert q.raw_call("qmv_packed_bytes", 0, 4, 32, 1, ctypes.byref(out)) == -2
    assert q.raw_call("qmv_packed_bytes", 1, 0, 32, 1, ctypes.byref(out)) == -4
    assert q.raw_call("qmv_packed_bytes", 1, 4, 33, 1, ctypes.byref(out)) == -4
    assert "multiple" in q.last_error()
    assert q.raw_call("qmv_packed_bytes", 3, 4, 128, 1, ctypes.byref(out)) == -4
    assert q.raw_call("qmv_packed_bytes", 1, 4, 32, 0, ctypes.byref(out)) == -4
    assert q.raw_call("qmv_packed_bytes", 1, 4, 32, 1, None) == -1
    assert q.raw_call("qmv_packed_bytes", 1, 1 << 40, 1 << 40, 1, ctypes.byref(out)) == -7


def test_matvec_argument_errors_before_any_launch(q):
    # fake, aligned, never dereferenced pointers: every case fails on the host
    P = 1 << 20
    F32, F16, BF16 = 1, 2, 3
    call = lambda *a: q.raw_call("qmv_matvec", *a)  # noqa: E731
    assert call(0, 8, 256, 1, P, P, F32, P, F32, None) == -2
    assert call(3, 8, 200, 1, P, P, F32, P, F32, None) == -4
    assert call(3, 8, 256, 0, P, P, F32, P, F32, None) == -4
    assert call(3, 8, 256, 1, None, P, F32, P, F32, None) == -1
    assert "W" in q.last_error()
    assert call(3, 8, 256, 1, P, None, F32, P, F32, None) == -1
    assert call(3, 8, 256, 1, P, P, 7, P, F32, None) == -6
    assert call(3, 8, 256, 1, P, P, F16, P, F32, None) == -3      # q4k takes f32 x
    assert call(2, 8, 256, 1, P, P, BF16, P, F32, None) == -3
    assert call(2, 8, 256, 1, P, P, F16, P, F16, None) == -3      # y is f32 only
    assert call(3, 8, 256, 1, P + 4, P, F32, P, F32, None) == -5
    assert call(3, 8, 256, 1, P, P + 8, F32, P, F32, None) == -5
    assert call(3, 8, 256, 1, P, P, F32, P + 2, F32, None) == -5


def test_gemm_and_pack_argument_errors(q):
    P = 1 << 20
    BF16 = 3
    assert q.raw_call("qmv_gemm", 3, 64, 256, 16, P, P, BF16, P, BF16, None) == -3
    assert "W4A16" in q.last_error()
    assert q.raw_call("qmv_gemm", 2, 64, 256, 16, P, P, 1, P, BF16, None) == -3
    assert q.raw_call("qmv_gemm", 2, 64, 100, 16, P, P, BF16, P, BF16, None) == -4
    assert q.raw_call("qmv_gemm", 2, 64, 256, 0, P, P, BF16, P, BF16, None) == -4
    src = q.QmvLogical()
    src.q = P
    assert q.raw_call("qmv_pack", 3, 8, 256, 1, ctypes.byref(src), P, None) == -1  # aux NULL
    assert "aux[0]" in q.last_error()
    for i in range(4):
        src.aux[i] = P
    assert q.raw_call("qmv_pack", 3, 8, 256, 1, None, P, None) == -1
    assert q.raw_call("qmv_pack", 3, 8, 256, 1, ctypes.byref(src), P + 8, None) == -5
    assert q.raw_call("qmv_dequant", 4, 8, 256, P, P + 4, None) == -5


def test_grouped_argument_errors(q):
    P = 1 << 20
    items = (q.QmvMatvecItem * 2)()
    for it in items:
        it.N, it.W, it.x, it.y = 64, P, P, P
    call = lambda *a: q.raw_call("qmv_matvec_grouped", *a)  # noqa: E731
    assert call(3, 256, 1, 0, items, 1, 1, None) == -4
    assert call(3, 256, 1, 2, None, 1, 1, None) == -1
    items[1].W = None
    assert call(3, 256, 1, 2, items, 1, 1, None) == -1
    assert "items[1].W" in q.last_error()
    items[1].W = P + 8
    assert call(3, 256, 1, 2, items, 1, 1, None) == -5
    items[1].W, items[1].N = P, 0
    assert call(3, 256, 1, 2, items, 1, 1, None) == -4
    items[1].N = 64
    assert call(3, 200, 1, 2, items, 1, 1, None) == -4
    assert call(3, 256, 1, 2, items, 2, 1, None) == -3
    assert call(3, 256, 1, 4097, items, 1, 1, None) == -4


def test_grouped_item_format_errors(q):
    # each item's format is its own fmt field, or the call's where that is 0
    assert ctypes.sizeof(q.QmvMatvecItem) == 40
    P = 1 << 20
    items = (q.QmvMatvecItem * 3)()
    for it in items:
        it.N, it.W, it.x, it.y, it.fmt = 64, P, P, P, 0
    call = lambda *a: q.raw_call("qmv_matvec_grouped", *a)  # noqa: E731
    assert call(0, 256, 1, 3, items, 1, 1, None) == -2  # no format anywhere
    assert "items[0].fmt" in q.last_error()
    items[0].fmt = items[1].fmt = 3
    assert call(0, 256, 1, 3, items, 1, 1, None) == -2
    assert "items[2]" in q.last_error()
    items[2].fmt = 10
    assert call(4, 256, 1, 3, items, 1, 1, None) == -2
    items[2].fmt = 2  # W4A16 beside Q4K: f16 activations suit only the W4A16 item
    assert call(0, 256, 1, 3, items, 2, 1, None) == -3
    assert "items[0]" in q.last_error()
    assert call(0, 64, 1, 3, items, 1, 1, None) == -4  # K = 64 is no Q4K block multiple
    assert "Q4K" in q.last_error() or "q4k" in q.last_error().lower()


def test_epilogue_and_swiglu_argument_errors(q):
    P = 1 << 20
    ep = q.QmvEpilogue()
    ex = lambda *a: q.raw_call("qmv_matvec_ex", *a)  # noqa: E731
    sw = lambda *a: q.raw_call("qmv_matvec_swiglu", *a)  # noqa: E731
    ep.bias = P + 2
    assert ex(3, 64, 256, 1, P, P, 1, P, 1, ctypes.byref(ep), None) == -5
    assert "bias" in q.last_error()
    ep.bias, ep.residual = P, P + 1
    assert ex(3, 64, 256, 1, P, P, 1, P, 1, ctypes.byref(ep), None) == -5
    assert "residual" in q.last_error()
    assert ex(3, 64, 200, 1, P, P, 1, P, 1, None, None) == -4    # K not a Q4K block multiple
    assert ex(11, 64, 256, 1, P, P, 1, P, 1, None, None) == -2   # no such format
    assert sw(3, 64, 256, 1, None, P, P, 1, P, 1, None) == -1
    assert "W_gate" in q.last_error()
    assert sw(3, 64, 256, 1, P, None, P, 1, P, 1, None) == -1
    assert "W_up" in q.last_error()
    assert sw(3, 64, 256, 1, P, P + 8, P, 1, P, 1, None) == -5
    assert "W_up" in q.last_error()
    assert sw(3, 64, 256, 1, P, P, P, 2, P, 1, None) == -3      # f16 x for Q4K


def test_q8x_sizes_and_errors(q):
    for K, b in ((32, 1), (96, 3), (2048, 8), (5632, 11)):
        assert q.q8x_bytes(K, b) == b * oracle.q8x_record_bytes(K)
    out = ctypes.c_size_t(0)
    assert q.raw_call("qmv_q8x_bytes", 48, 1, ctypes.byref(out)) == -4
    assert q.raw_call("qmv_q8x_bytes", 64, 0, ctypes.byref(out)) == -4
    assert q.raw_call("qmv_q8x_bytes", 64, 1, None) == -1
    P = 1 << 20
    assert q.raw_call("qmv_quantize_x", 64, 1, None, P, None) == -1
    assert q.raw_call("qmv_quantize_x", 64, 1, P, P + 4, None) == -5
    # Q8X activations: any integer-code format, not dense bf16
    assert q.raw_call("qmv_matvec", 8, 64, 256, 1, P, P, 4, P, 1, None) == -3
    assert "DENSE_BF16" in q.last_error()
