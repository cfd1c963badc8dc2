"""Python binding of libqmv: fused dequantize-and-multiply of block-quantized
weights on MI355X (gfx950).

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of libqmv.so; PyTorch supplies device memory and the current stream.
Importing this package fails loudly when the library has not been built
(`python gemm_dequant_matvec_amd/build.py`); there is no CPU fallback.

    import gemm_dequant_matvec_amd as qmv
    W = qmv.pack("q4k", {"q": q, "sc": sc, "m": m, "d": d, "dmin": dmin})
    y = qmv.matvec("q4k", W, x, N, K)          # x [b][K] f32 -> y [b][N] f32
    Y = qmv.gemm("w4a16_g64", W, X, N, K)      # X [M][K] bf16 -> Y [M][N] bf16
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmv.so")

FORMATS = {"q8_0": 1, "w4a16_g64": 2, "q4k": 3, "q6k": 4, "q4_0": 5, "q5_0": 6, "q5k": 7, "bf16": 8,
           "i8row": 9}
BLOCK = {"q8_0": 32, "w4a16_g64": 64, "q4k": 256, "q6k": 256, "q4_0": 32, "q5_0": 32, "q5k": 256, "bf16": 32,
         "i8row": 32}
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
_DTYPES = {torch.float32: 1, torch.float16: 2, torch.bfloat16: 3}
# (weights per element, bytes per element) of each logical aux array
_AUX_SHAPE = {
    "q8_0": {"scale": (32, 2)},
    "w4a16_g64": {"scale": (64, 2), "zero": (64, 2)},
    "q4k": {"sc": (32, 1), "m": (32, 1), "d": (256, 2), "dmin": (256, 2)},
    "q6k": {"s": (16, 1), "d": (256, 2)},
    "q4_0": {"d": (32, 2)},
    "q5_0": {"d": (32, 2)},
    "q5k": {"sc": (32, 1), "m": (32, 1), "d": (256, 2), "dmin": (256, 2)},
    "i8row": {"scale": (None, 4)},  # one per row
}

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libqmv.so not found at {LIB_PATH}: build it with "
        "`python gemm_dequant_matvec_amd/build.py` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)


class QmvLogical(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("aux", ctypes.c_void_p * 4)]


_i64, _vp, _int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
_lib.qmv_abi_version.argtypes = [ctypes.POINTER(ctypes.c_int)]
_lib.qmv_abi_version.restype = _int
_lib.qmv_status_string.argtypes = [_int]
_lib.qmv_status_string.restype = ctypes.c_char_p
_lib.qmv_last_error.argtypes = []
_lib.qmv_last_error.restype = ctypes.c_char_p
_lib.qmv_packed_bytes.argtypes = [_int, _i64, _i64, _i64, ctypes.POINTER(ctypes.c_size_t)]
_lib.qmv_packed_bytes.restype = _int
_lib.qmv_pack.argtypes = [_int, _i64, _i64, _i64, ctypes.POINTER(QmvLogical), _vp, _vp]
_lib.qmv_pack.restype = _int
_lib.qmv_matvec.argtypes = [_int, _i64, _i64, _i64, _vp, _vp, _int, _vp, _int, _vp]
_lib.qmv_matvec.restype = _int


class QmvEpilogue(ctypes.Structure):
    _fields_ = [("bias", ctypes.c_void_p), ("residual", ctypes.c_void_p)]


_lib.qmv_matvec_ex.argtypes = [_int, _i64, _i64, _i64, _vp, _vp, _int, _vp, _int, ctypes.POINTER(QmvEpilogue), _vp]
_lib.qmv_matvec_ex.restype = _int
_lib.qmv_matvec_swiglu.argtypes = [_int, _i64, _i64, _i64, _vp, _vp, _vp, _int, _vp, _int, _vp]
_lib.qmv_matvec_swiglu.restype = _int


class QmvMatvecItem(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("W", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("fmt", ctypes.c_int32)]


_lib.qmv_matvec_grouped.argtypes = [_int, _i64, _i64, _int, ctypes.POINTER(QmvMatvecItem), _int, _int, _vp]
_lib.qmv_matvec_grouped.restype = _int
_lib.qmv_quantize_x.argtypes = [_i64, _i64, _vp, _vp, _vp]
_lib.qmv_quantize_x.restype = _int
_lib.qmv_q8x_bytes.argtypes = [_i64, _i64, ctypes.POINTER(ctypes.c_size_t)]
_lib.qmv_q8x_bytes.restype = _int
_lib.qmv_gemm.argtypes = [_int, _i64, _i64, _i64, _vp, _vp, _int, _vp, _int, _vp]
_lib.qmv_gemm.restype = _int
_lib.qmv_dequant.argtypes = [_int, _i64, _i64, _vp, _vp, _vp]
_lib.qmv_dequant.restype = _int

EXPORTS = ("qmv_abi_version", "qmv_status_string", "qmv_last_error", "qmv_packed_bytes",
           "qmv_pack", "qmv_matvec", "qmv_matvec_ex", "qmv_matvec_swiglu", "qmv_matvec_grouped", "qmv_gemm",
           "qmv_dequant", "qmv_quantize_x", "qmv_q8x_bytes")


class QmvError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{_lib.qmv_status_string(status).decode()} ({status}): {message}")


def _check(status: int) -> None:
    if status != 0:
        raise QmvError(status, _lib.qmv_last_error().decode())


def _fmt(fmt) -> int:
    if isinstance(fmt, str):
        if fmt not in FORMATS:
            raise ValueError(f"unknown format {fmt!r}; one of {sorted(FORMATS)}")
        return FORMATS[fmt]
    return int(fmt)


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _need(t: torch.Tensor, nbytes: int, what: str) -> None:
    """The C ABI sees only pointers: a buffer shorter than the call will touch
    is rejected here, before anything reaches the device."""
    if _nbytes(t) < nbytes:
        raise ValueError(f"{what} holds {_nbytes(t)} bytes, the call needs {nbytes}")


def _need_dtype(t: torch.Tensor, dtype: torch.dtype, what: str) -> None:
    if t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype}, got {t.dtype}")


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to libqmv must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libqmv must be contiguous")
    return t.data_ptr()


def abi_version() -> tuple[int, int]:
    lv = ctypes.c_int(0)
    v = _lib.qmv_abi_version(ctypes.byref(lv))
    return v, lv.value


def packed_bytes(fmt, N: int, K: int, batch: int = 1) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.qmv_packed_bytes(_fmt(fmt), N, K, batch, ctypes.byref(out)))
    return out.value


def pack(fmt, logical: dict, N: int | None = None, K: int | None = None, batch: int = 1,
         out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Pack logical device arrays (dict of tensors named as in AUX_FIELDS plus "q")."""
    name = fmt if isinstance(fmt, str) else {v: k for k, v in FORMATS.items()}[fmt]
    q = logical["q"]
    if N is None or K is None:
        N, K = q.shape[-2], q.shape[-1]
    nbytes = packed_bytes(name, N, K, batch)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    _need(out, nbytes, "out")
    _need(q, batch * N * K * (2 if name == "bf16" else 1), "q")
    for field in AUX_FIELDS[name]:
        if field not in logical:
            raise ValueError(f"{name} needs the logical array {field!r}")
        per = _AUX_SHAPE[name][field]
        _need(logical[field], batch * N * (K // per[0] if per[0] else 1) * per[1], field)
    src = QmvLogical()
    src.q = _ptr(q)
    for i, field in enumerate(AUX_FIELDS[name]):
        src.aux[i] = _ptr(logical[field])
    _check(_lib.qmv_pack(_fmt(name), N, K, batch, ctypes.byref(src), _ptr(out), _stream(stream)))
    return out


class Q8X:
    """Activations quantized to 8-bit blocks by quantize_x: `data` is the
    device buffer (uint8), `K` and `batch` its shape."""

    def __init__(self, data: torch.Tensor, K: int, batch: int):
        self.data, self.K, self.batch = data, K, batch


def q8x_bytes(K: int, batch: int) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.qmv_q8x_bytes(K, batch, ctypes.byref(out)))
    return out.value


def quantize_x(x: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> Q8X:
    """f32 x [b][K] -> Q8X (per 32 activations: 8-bit codes and an f32 scale)."""
    x2 = x if x.dim() == 2 else x.reshape(1, -1)
    b, K = x2.shape
    nbytes = q8x_bytes(K, b)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    _need_dtype(x2, torch.float32, "x")
    _need(out, nbytes, "out")
    _check(_lib.qmv_quantize_x(K, b, _ptr(x2), _ptr(out), _stream(stream)))
    return Q8X(out, K, b)


def _xarg(x, K: int):
    """(pointer, dtype code, batch) of an activation argument: a tensor [b][K]
    (f32 / f16) or a Q8X."""
    if isinstance(x, Q8X):
        if x.K != K:
            raise ValueError(f"Q8X activations have K={x.K}, expected K={K}")
        _need(x.data, q8x_bytes(K, x.batch), "x")
        return _ptr(x.data), 4, x.batch, x.data.device
    x2 = x if x.dim() == 2 else x.reshape(1, -1)
    if x2.shape[1] != K:
        raise ValueError(f"x has {x2.shape[1]} columns, expected K={K}")
    if x2.dtype not in _DTYPES:
        raise ValueError("x dtype must be float32, float16 or bfloat16")
    return _ptr(x2), _DTYPES[x2.dtype], x2.shape[0], x2.device


def matvec(fmt, W: torch.Tensor, x, N: int, K: int, y: torch.Tensor | None = None,
           stream=None) -> torch.Tensor:
    """y [b][N] f32 = W x for x [b][K] (f32, f16 for w4a16_g64, or a Q8X from quantize_x)."""
    b = x.batch if isinstance(x, Q8X) else (x.shape[0] if x.dim() == 2 else 1)
    dev = x.data.device if isinstance(x, Q8X) else x.device
    if y is None:
        y = torch.empty((b, N), dtype=torch.float32, device=dev)
    if y.dtype not in _DTYPES:
        raise ValueError("y dtype must be float32, float16 or bfloat16")
    _need(W, packed_bytes(fmt, N, K), "W")
    _need(y, b * N * 4, "y")
    xp, xdt, b, _ = _xarg(x, K)
    _check(_lib.qmv_matvec(_fmt(fmt), N, K, b, _ptr(W), xp, xdt, _ptr(y), _DTYPES[y.dtype], _stream(stream)))
    return y


def matvec_ex(fmt, W: torch.Tensor, x: torch.Tensor, N: int, K: int, y: torch.Tensor | None = None,
              bias: torch.Tensor | None = None, residual: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y [b][N] f32 = residual + (W x + bias): the bias / residual add fused into
    the matvec.  bias f32 [N] or None; residual f32 [b][N] or None (may be y).
    x as in matvec."""
    b = x.batch if isinstance(x, Q8X) else (x.shape[0] if x.dim() == 2 else 1)
    dev = x.data.device if isinstance(x, Q8X) else x.device
    if y is None:
        y = torch.empty((b, N), dtype=torch.float32, device=dev)
    if y.dtype not in _DTYPES:
        raise ValueError("y dtype must be float32, float16 or bfloat16")
    _need(W, packed_bytes(fmt, N, K), "W")
    _need(y, b * N * 4, "y")
    if bias is not None:
        _need_dtype(bias, torch.float32, "bias")
        _need(bias, N * 4, "bias")
    if residual is not None:
        _need_dtype(residual, torch.float32, "residual")
        _need(residual, b * N * 4, "residual")
    xp, xdt, b, _ = _xarg(x, K)  # every size check above: pointers only from here on
    ep = QmvEpilogue()
    ep.bias = _ptr(bias)
    ep.residual = _ptr(residual)
    _check(_lib.qmv_matvec_ex(_fmt(fmt), N, K, b, _ptr(W), xp, xdt, _ptr(y),
                              _DTYPES[y.dtype], ctypes.byref(ep), _stream(stream)))
    return y


def matvec_swiglu(fmt, W_gate: torch.Tensor, W_up: torch.Tensor, x: torch.Tensor, N: int, K: int,
                  h: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """h [b][N] f32 = silu(W_gate x) * (W_up x), gate / up / SwiGLU in one pass
    (x as in matvec)."""
    b = x.batch if isinstance(x, Q8X) else (x.shape[0] if x.dim() == 2 else 1)
    dev = x.data.device if isinstance(x, Q8X) else x.device
    if h is None:
        h = torch.empty((b, N), dtype=torch.float32, device=dev)
    if h.dtype not in _DTYPES:
        raise ValueError("h dtype must be float32, float16 or bfloat16")
    _need(W_gate, packed_bytes(fmt, N, K), "W_gate")
    _need(W_up, packed_bytes(fmt, N, K), "W_up")
    _need(h, b * N * 4, "h")
    xp, xdt, b, _ = _xarg(x, K)
    _check(_lib.qmv_matvec_swiglu(_fmt(fmt), N, K, b, _ptr(W_gate), _ptr(W_up), xp, xdt,
                                  _ptr(h), _DTYPES[h.dtype], _stream(stream)))
    return h


def matvec_grouped(fmt, items, K: int, stream=None) -> list:
    """Several matvecs of one K in as few launches as possible.

    items: sequence of (W, x, N), (W, x, N, y) or (W, x, N, y, item_fmt); x
    [b][K] (same b and dtype for all) or a Q8X of b vectors (then for all), y
    allocated as f32 [b][N] when absent or None; item_fmt overrides fmt for
    that matrix (fmt may then be None).  Returns the list of y.
    """
    arr = (QmvMatvecItem * len(items))()
    outs, rows = [], []
    b = xdt = None
    for i, it in enumerate(items):  # every size check before any pointer is taken
        W, x, N = it[0], it[1], it[2]
        if isinstance(x, Q8X):
            if x.K != K:
                raise ValueError(f"items[{i}]: Q8X activations have K={x.K}, expected K={K}")
            _need(x.data, q8x_bytes(K, x.batch), f"items[{i}].x")
            x2, shape, dt, device = x.data, (x.batch, K), "q8x", x.data.device
        else:
            x2 = x if x.dim() == 2 else x.reshape(1, -1)
            shape, dt, device = tuple(x2.shape), x2.dtype, x.device
            if dt not in _DTYPES:
                raise ValueError("x dtype must be float32, float16 or bfloat16")
        if b is None:
            b, xdt = shape[0], dt
        if shape != (b, K) or dt != xdt:
            raise ValueError("all items need x of shape [b][K] and one dtype")
        y = it[3] if len(it) > 3 and it[3] is not None else torch.empty((b, N), dtype=torch.float32,
                                                                          device=device)
        ifmt = it[4] if len(it) > 4 and it[4] is not None else fmt
        if ifmt is None:
            raise ValueError(f"item {i} names no format and the call's fmt is None")
        _need(W, packed_bytes(ifmt, N, K), f"items[{i}].W")
        _need(y, b * N * 4, f"items[{i}].y")
        rows.append((W, x2, N, y, it[4] if len(it) > 4 else None))
        outs.append(y)
    for i, (W, x2, N, y, ifmt) in enumerate(rows):
        arr[i].N, arr[i].W, arr[i].x, arr[i].y = N, _ptr(W), _ptr(x2), _ptr(y)
        arr[i].fmt = _fmt(ifmt) if ifmt is not None else 0
    _check(_lib.qmv_matvec_grouped(0 if fmt is None else _fmt(fmt), K, b, len(items), arr,
                                   4 if xdt == "q8x" else _DTYPES[xdt],
                                   _DTYPES[torch.float32], _stream(stream)))
    return outs


def gemm(fmt, W: torch.Tensor, X: torch.Tensor, N: int, K: int, Y: torch.Tensor | None = None,
         stream=None) -> torch.Tensor:
    """Y [M][N] bf16 = X W^T for X [M][K] bf16, on the matrix cores."""
    M = X.shape[0]
    if X.shape[1] != K:
        raise ValueError(f"X has {X.shape[1]} columns, expected K={K}")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    if X.dtype not in _DTYPES or Y.dtype not in _DTYPES:
        raise ValueError("X / Y dtype must be float32, float16 or bfloat16")
    _need(W, packed_bytes(fmt, N, K), "W")
    _need(Y, M * N * Y.element_size(), "Y")
    _check(_lib.qmv_gemm(_fmt(fmt), N, K, M, _ptr(W), _ptr(X), _DTYPES[X.dtype], _ptr(Y),
                         _DTYPES[Y.dtype], _stream(stream)))
    return Y


def dequant(fmt, W: torch.Tensor, N: int, K: int, out: torch.Tensor | None = None,
            stream=None) -> torch.Tensor:
    """Dense f32 [N][K] copy of a packed matrix (bit-exact; inspection/testing)."""
    if out is None:
        out = torch.empty((N, K), dtype=torch.float32, device=W.device)
    _need(W, packed_bytes(fmt, N, K), "W")
    _need_dtype(out, torch.float32, "out")
    _need(out, N * K * 4, "out")
    _check(_lib.qmv_dequant(_fmt(fmt), N, K, _ptr(W), _ptr(out), _stream(stream)))
    return out


def raw_call(name: str, *args) -> int:
    """Call a C entry point with raw arguments (tests of the ABI's error paths)."""
    return getattr(_lib, name)(*args)


def last_error() -> str:
    return _lib.qmv_last_error().decode()
