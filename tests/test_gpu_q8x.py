"""GPU parity of the integer-dot variant: activations quantized to 8-bit blocks
(qmv_quantize_x) and the matvec over them (x_dtype QMV_Q8X).

The pages' CPU decode path quantizes the activation vector once per matmul
and computes every row as integer dot products scaled back to f32 (aot-llm
README, How it works).  Bars:
  * the quantizer: codes and scales bit-exact against the oracle's
    quantize_q8x, including ties, all-zero and tiny blocks;
  * the matvec: within 1e-3 * ||W_row|| * ||x^|| of the f64 product of the
    exact dequantized weights and the quantized activations x^ = d q (the
    oracle's buffer is the input, so this does not lean on the quantizer);
  * against the unquantized f32 x the result also carries the quantization
    error, bounded per element by |x - x^| <= 0.51 d of its block.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_helpers import dev, pack_dev

pytestmark = pytest.mark.gpu

TAU = oracle.reference.TAU_F32
INT_FORMATS = ["q8_0", "w4a16_g64", "q4k", "q6k", "q4_0", "q5_0", "q5k", "i8row"]
SHAPES = [(130, 512), (200, 1024), (129, 2048), (70, 5632)]


def _say(*a):
    print(*a, flush=True)


def _special_x(K, b, key):
    """Seeded N(0,1)-like activations with hand-made blocks in vector 0:
    all zero, a ramp, exact ties, a tiny block, the 2^-120 threshold, huge values."""
    x = wl.gen_x(K, b, "f32", key).astype(np.float32)
    nblk = K // 32
    k = np.arange(32, dtype=np.float32)
    blocks = [np.zeros(32, np.float32), 0.25 * (k - 16),
              np.array([127, 2.5, 3.5, -2.5, -0.5, 0.5] + [0] * 26, np.float32),
              np.array([1e-37, -5e-38] + [0] * 30, np.float32),
              np.array([2.0 ** -120, -(2.0 ** -121)] + [0] * 30, np.float32),
              np.float32(1e30) * np.sin(k)]
    for j, blk in enumerate(blocks[:nblk]):
        x[0, 32 * j:32 * j + 32] = blk
    return x


def _record_bytes(buf: np.ndarray, K: int, b: int) -> np.ndarray:
    rec = oracle.q8x_record_bytes(K)
    return np.stack([buf[i * rec:i * rec + K + K // 8] for i in range(b)])


@pytest.mark.parametrize("K,b", [(32, 1), (96, 3), (2048, 8), (5632, 11), (14336, 2), (2048, 64)])
def test_quantize_bit_exact(qmv, K, b):
    _say("quantize", K, b)
    x = _special_x(K, b, (71, K, b))
    xq = qmv.quantize_x(dev(x))
    torch.cuda.synchronize()
    got = _record_bytes(xq.data.cpu().numpy(), K, b)
    want = _record_bytes(oracle.pack_q8x(*oracle.quantize_q8x(x)), K, b)
    assert np.array_equal(got, want), np.argwhere(got != want)[:8]


def _q8x_input(x):
    q, d = oracle.quantize_q8x(x)
    return q, d, dev(oracle.pack_q8x(q, d))


@pytest.mark.parametrize("fmt", INT_FORMATS)
@pytest.mark.parametrize("batch", [1, 3, 8, 11])
def test_q8x_matvec_parity(qmv, fmt, batch):
    for N, K in SHAPES:
        if K % wl.BLOCK[fmt]:
            continue
        _say("q8x matvec", fmt, N, K, batch)
        key = (72, N, K)
        w = wl.gen_weights(fmt, N, K, key)
        x = wl.gen_x(K, batch, "f32", key)
        q, d, buf = _q8x_input(x)
        Wp = pack_dev(qmv, fmt, w)
        y = qmv.matvec(fmt, Wp, qmv.Q8X(buf, K, batch), N, K)
        torch.cuda.synchronize()
        y = y.cpu().numpy()
        W32 = oracle.dequant(fmt, w)
        xh = oracle.dequant_q8x(q, d)
        bound = oracle.tolerance_bound(W32, xh, TAU)
        r = oracle.check_within(y, oracle.matvec_ref(W32, xh), bound)
        assert r["ok"], (fmt, N, K, batch, r)
        # against the f32 activations: plus the quantization error of x
        qerr = np.abs(W32.astype(np.float64)) @ (0.51 * np.repeat(d.astype(np.float64), 32, axis=1)).T
        r2 = oracle.check_within(y, oracle.matvec_ref(W32, x.astype(np.float64)), bound + qerr.T)
        assert r2["ok"], (fmt, N, K, batch, r2)


@pytest.mark.parametrize("fmt", ["q4k", "q6k", "q8_0"])
def test_quantize_then_matvec_end_to_end(qmv, fmt):
    N, K, batch = 300, 2048, 4
    w = wl.gen_weights(fmt, N, K, (73, N, K))
    x = wl.gen_x(K, batch, "f32", (73, N, K))
    Wp = pack_dev(qmv, fmt, w)
    y = qmv.matvec(fmt, Wp, qmv.quantize_x(dev(x)), N, K)
    torch.cuda.synchronize()
    q, d = oracle.quantize_q8x(x)
    W32 = oracle.dequant(fmt, w)
    xh = oracle.dequant_q8x(q, d)
    r = oracle.check_within(y.cpu().numpy(), oracle.matvec_ref(W32, xh), oracle.tolerance_bound(W32, xh, TAU))
    assert r["ok"], r


@pytest.mark.parametrize("fmt", ["q4k", "q6k", "i8row", "q5_0"])
@pytest.mark.parametrize("batch", [1, 8])
def test_q8x_epilogue_and_swiglu(qmv, fmt, batch):
    N, K = 200, 1024
    wg = wl.gen_weights(fmt, N, K, (74, N, K))
    wu = wl.gen_weights(fmt, N, K, (75, N, K))
    x = wl.gen_x(K, batch, "f32", (74, N, K))
    q, d, buf = _q8x_input(x)
    xh = oracle.dequant_q8x(q, d)
    xq = qmv.Q8X(buf, K, batch)
    G, U = oracle.dequant(fmt, wg), oracle.dequant(fmt, wu)
    g, dg = oracle.matvec_ref(G, xh), oracle.tolerance_bound(G, xh, TAU)
    u, du = oracle.matvec_ref(U, xh), oracle.tolerance_bound(U, xh, TAU)
    Wg, Wu = pack_dev(qmv, fmt, wg), pack_dev(qmv, fmt, wu)
    _say("q8x swiglu", fmt, batch)
    h = qmv.matvec_swiglu(fmt, Wg, Wu, xq, N, K)
    torch.cuda.synchronize()
    r = oracle.check_within(h.cpu().numpy(), oracle.swiglu_ref(g, u), oracle.swiglu_bound(g, u, dg, du))
    assert r["ok"], r
    rng = np.random.default_rng(batch)
    bias = rng.normal(0, 1, N).astype(np.float32)
    res = rng.normal(0, 3, (batch, N)).astype(np.float32)
    _say("q8x epilogue", fmt, batch)
    out = qmv.matvec_ex(fmt, Wg, xq, N, K, bias=dev(bias), residual=dev(res))
    torch.cuda.synchronize()
    r = oracle.check_within(out.cpu().numpy(), oracle.epilogue_ref(g, bias, res),
                            oracle.epilogue_bound(dg, g, bias, res))
    assert r["ok"], r


@pytest.mark.parametrize("batch", [1, 5])
def test_q8x_grouped_mixed_formats(qmv, batch):
    K = 2048
    x = wl.gen_x(K, batch, "f32", (76, 0, K))
    q, d, buf = _q8x_input(x)
    xh = oracle.dequant_q8x(q, d)
    xq = qmv.Q8X(buf, K, batch)
    specs = [("q4k", 256), ("q6k", 130), ("q8_0", 64), ("w4a16_g64", 70)]
    ws = [wl.gen_weights(f, n, K, (76, n, i)) for i, (f, n) in enumerate(specs)]
    items = [(pack_dev(qmv, f, w), xq, n, None, f) for (f, n), w in zip(specs, ws)]
    _say("q8x grouped", batch)
    ys = qmv.matvec_grouped(None, items, K)
    torch.cuda.synchronize()
    for (f, n), w, y in zip(specs, ws, ys):
        W32 = oracle.dequant(f, w)
        r = oracle.check_within(y.cpu().numpy(), oracle.matvec_ref(W32, xh), oracle.tolerance_bound(W32, xh, TAU))
        assert r["ok"], (f, n, r)


def test_q8x_rejects_dense_bf16(qmv):
    N, K = 64, 256
    w = wl.gen_weights("bf16", N, K, (77, 0, 0))
    x = wl.gen_x(K, 1, "f32", (77, 0, 0))
    with pytest.raises(qmv.QmvError, match="DENSE_BF16"):
        qmv.matvec("bf16", pack_dev(qmv, "bf16", w), qmv.quantize_x(dev(x)), N, K)


@pytest.mark.parametrize("fmt,N,K", [("q4k", 5632, 2048), ("q6k", 2048, 5632), ("w4a16_g64", 5632, 2048),
                                     ("q8_0", 1, 32), ("q5k", 17, 256), ("i8row", 3, 64)])
@pytest.mark.parametrize("batch", [1, 8])
def test_q8x_matvec_sizes(qmv, fmt, N, K, batch):
    # the decoder's gate / down shapes (every row), and one row, 17 rows, one block of K
    _say("q8x sizes", fmt, N, K, batch)
    w = wl.gen_weights(fmt, N, K, (78, N, K))
    x = wl.gen_x(K, batch, "f32", (78, N, K))
    q, d, buf = _q8x_input(x)
    y = qmv.matvec(fmt, pack_dev(qmv, fmt, w), qmv.Q8X(buf, K, batch), N, K)
    torch.cuda.synchronize()
    W32 = oracle.dequant(fmt, w)
    xh = oracle.dequant_q8x(q, d)
    r = oracle.check_within(y.cpu().numpy(), oracle.matvec_ref(W32, xh), oracle.tolerance_bound(W32, xh, TAU))
    assert r["ok"], r
