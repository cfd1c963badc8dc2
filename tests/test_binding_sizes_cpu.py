"""The Python binding rejects buffers shorter than a call would touch (no GPU).

The C ABI receives bare pointers and cannot see buffer sizes, so the binding
is the only layer that can check them.  Every check runs before any pointer
is taken, so CPU tensors exercise it here; a correctly sized CPU tensor then
fails the device check instead.
"""
import pytest
import torch

import gemm_dequant_matvec_amd as qmv


def _u8(n):
    return torch.zeros(n, dtype=torch.uint8)


@pytest.mark.parametrize("fmt", sorted(qmv.FORMATS))
def test_matvec_short_w_and_y(fmt):
    N, K = 64, 512
    need = qmv.packed_bytes(fmt, N, K)
    x = torch.zeros((1, K), dtype=torch.float32)
    with pytest.raises(ValueError, match="W holds"):
        qmv.matvec(fmt, _u8(need - 1), x, N, K, y=torch.zeros((1, N)))
    with pytest.raises(ValueError, match="y holds"):
        qmv.matvec(fmt, _u8(need), x, N, K, y=torch.zeros((1, N - 1)))
    with pytest.raises(ValueError, match="y holds"):  # batch 2 needs two rows of y
        qmv.matvec(fmt, _u8(need), torch.zeros((2, K)), N, K, y=torch.zeros((1, N)))
    with pytest.raises(ValueError, match="GPU"):  # sizes fine: only the device check is left
        qmv.matvec(fmt, _u8(need), x, N, K, y=torch.zeros((1, N)))


def test_grouped_short_buffers_name_the_item():
    K = 256
    need = qmv.packed_bytes("q4k", 32, K)
    x = torch.zeros((1, K))
    good = (_u8(need), x, 32, torch.zeros((1, 32)))
    with pytest.raises(ValueError, match=r"items\[1\]\.W"):
        qmv.matvec_grouped("q4k", [good, (_u8(need - 16), x, 32, torch.zeros((1, 32)))], K)
    with pytest.raises(ValueError, match=r"items\[1\]\.y"):
        qmv.matvec_grouped("q4k", [good, (_u8(need), x, 32, torch.zeros((1, 31)))], K)
    # an item whose own format needs more bytes than the call's format
    need6 = qmv.packed_bytes("q6k", 32, K)
    assert need6 > need
    with pytest.raises(ValueError, match=r"items\[0\]\.W"):
        qmv.matvec_grouped("q4k", [(_u8(need), x, 32, torch.zeros((1, 32)), "q6k")], K)


def test_gemm_short_w_and_y():
    N, K, M = 128, 256, 5
    need = qmv.packed_bytes("w4a16_g64", N, K)
    X = torch.zeros((M, K), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="W holds"):
        qmv.gemm("w4a16_g64", _u8(need - 1), X, N, K, Y=torch.zeros((M, N), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="Y holds"):
        qmv.gemm("w4a16_g64", _u8(need), X, N, K, Y=torch.zeros((M - 1, N), dtype=torch.bfloat16))


def test_dequant_short_or_wrong_out():
    N, K = 8, 64
    need = qmv.packed_bytes("q8_0", N, K)
    with pytest.raises(ValueError, match="W holds"):
        qmv.dequant("q8_0", _u8(need - 1), N, K, out=torch.zeros((N, K)))
    with pytest.raises(ValueError, match="out holds"):
        qmv.dequant("q8_0", _u8(need), N, K, out=torch.zeros((N, K - 1)))
    with pytest.raises(ValueError, match="out must be"):
        qmv.dequant("q8_0", _u8(need), N, K, out=torch.zeros((N, K), dtype=torch.float16))


def test_pack_short_logical_arrays_and_out():
    N, K = 16, 256
    lg = {"q": _u8(N * K), "sc": _u8(N * K // 32), "m": _u8(N * K // 32),
          "d": torch.zeros(N * K // 256, dtype=torch.int16), "dmin": torch.zeros(N * K // 256, dtype=torch.int16)}
    need = qmv.packed_bytes("q4k", N, K)
    with pytest.raises(ValueError, match="out holds"):
        qmv.pack("q4k", lg, N, K, out=_u8(need - 1))
    for field in ("q", "sc", "m", "d", "dmin"):
        bad = dict(lg)
        bad[field] = lg[field][:-1]
        with pytest.raises(ValueError, match=f"{field} holds"):
            qmv.pack("q4k", bad, N, K, out=_u8(need))
    missing = {k: v for k, v in lg.items() if k != "dmin"}
    with pytest.raises(ValueError, match="dmin"):
        qmv.pack("q4k", missing, N, K, out=_u8(need))
    with pytest.raises(ValueError, match="q holds"):  # two stacked matrices need twice the codes
        qmv.pack("q4k", lg, N, K, batch=2, out=_u8(2 * need))


def test_epilogue_short_buffers():
    N, K, b = 64, 256, 3
    need = qmv.packed_bytes("q4k", N, K)
    x = torch.zeros((b, K))
    y = torch.zeros((b, N))
    with pytest.raises(ValueError, match="bias holds"):
        qmv.matvec_ex("q4k", _u8(need), x, N, K, y=y, bias=torch.zeros(N - 1), residual=torch.zeros((b, N)))
    with pytest.raises(ValueError, match="residual holds"):
        qmv.matvec_ex("q4k", _u8(need), x, N, K, y=y, bias=torch.zeros(N), residual=torch.zeros((b - 1, N)))
    with pytest.raises(ValueError, match="bias must be"):
        qmv.matvec_ex("q4k", _u8(need), x, N, K, y=y, bias=torch.zeros(N, dtype=torch.float16))
    with pytest.raises(ValueError, match="GPU"):
        qmv.matvec_ex("q4k", _u8(need), x, N, K, y=y, bias=torch.zeros(N), residual=torch.zeros((b, N)))
    with pytest.raises(ValueError, match="W_up holds"):
        qmv.matvec_swiglu("q4k", _u8(need), _u8(need - 1), x, N, K, h=y)
    with pytest.raises(ValueError, match="h holds"):
        qmv.matvec_swiglu("q4k", _u8(need), _u8(need), x, N, K, h=torch.zeros((b, N - 1)))


def test_q8x_short_buffers():
    K, b = 256, 2
    nbytes = qmv.q8x_bytes(K, b)
    assert nbytes == b * ((K + K // 8 + 15) // 16 * 16)
    with pytest.raises(ValueError, match="out holds"):
        qmv.quantize_x(torch.zeros((b, K)), out=_u8(nbytes - 1))
    with pytest.raises(ValueError, match="x must be"):
        qmv.quantize_x(torch.zeros((b, K), dtype=torch.float16), out=_u8(nbytes))
    N = 32
    need = qmv.packed_bytes("q6k", N, K)
    with pytest.raises(ValueError, match="x holds"):
        qmv.matvec("q6k", _u8(need), qmv.Q8X(_u8(nbytes - 16), K, b), N, K, y=torch.zeros((b, N)))
    with pytest.raises(ValueError, match="K=512"):
        qmv.matvec("q6k", _u8(qmv.packed_bytes("q6k", N, 512)), qmv.Q8X(_u8(nbytes), K, b), N, 512,
                   y=torch.zeros((b, N)))
    with pytest.raises(ValueError, match="GPU"):
        qmv.matvec("q6k", _u8(need), qmv.Q8X(_u8(nbytes), K, b), N, K, y=torch.zeros((b, N)))
