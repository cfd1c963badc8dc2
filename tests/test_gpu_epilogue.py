"""GPU parity of the fused decode epilogues against the CPU oracle.

qmv_matvec_ex adds a bias and a residual in the matvec's epilogue;
qmv_matvec_swiglu computes silu(W_gate x) * (W_up x) in one pass over both
matrices (aot-llm README, Metal backend notes).  References: the oracle's
epilogue_ref / swiglu_ref in f64 over the exact dequantized weights, with
the matvec bound propagated (epilogue_bound, swiglu_bound).  Shapes reach
the streaming kernel's lanes-per-row settings (16 / 32 / 64 lanes, K split
over waves) at batch 1, and at batch 2..11 the matrix-core kernel (Q8_0,
W4A16, Q4K, Q6K: one to eleven waves per workgroup, one or two K chunks per
wave) or the FMA kernel (the other formats).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_helpers import dev, dev_x, pack_dev, x_values

pytestmark = pytest.mark.gpu

XDT = {"w4a16_g64": "f16"}
TAU = oracle.reference.TAU_F32


def _say(*a):
    print(*a, flush=True)


def _prod(fmt, w, x, xd):
    W32 = oracle.dequant(fmt, w)
    xv = x_values(x, xd)
    return oracle.matvec_ref(W32, xv), oracle.tolerance_bound(W32, xv, TAU)


SHAPES = [(100, 256), (130, 512), (200, 1024), (129, 2048), (70, 5632)]


@pytest.mark.parametrize("fmt", ["q4k", "q6k", "w4a16_g64", "q8_0", "q5k", "i8row"])
@pytest.mark.parametrize("batch", [1, 3, 8, 9])
def test_bias_and_residual_epilogue(qmv, fmt, batch):
    for N, K in SHAPES:
        if K % wl.BLOCK[fmt]:
            continue
        xd = XDT.get(fmt, "f32")
        key = (61, N, K)
        w = wl.gen_weights(fmt, N, K, key)
        x = wl.gen_x(K, batch, xd, key)
        g = np.random.default_rng(N + K + batch)
        bias = g.normal(0, 1, N).astype(np.float32)
        res = g.normal(0, 3, (batch, N)).astype(np.float32)
        Wp = pack_dev(qmv, fmt, w)
        ymv, bmv = _prod(fmt, w, x, xd)
        for case in ("bias", "residual", "both", "in-place"):
            _say(fmt, N, K, batch, case)
            bd = dev(bias) if case in ("bias", "both") else None
            rd = dev(res) if case in ("residual", "both", "in-place") else None
            y = rd if case == "in-place" else None
            out = qmv.matvec_ex(fmt, Wp, dev_x(x, xd), N, K, y=y, bias=bd, residual=rd)
            torch.cuda.synchronize()
            bb = bias if bd is not None else None
            rr = res if rd is not None else None
            ref = oracle.epilogue_ref(ymv, bb, rr)
            r = oracle.check_within(out.cpu().numpy(), ref, oracle.epilogue_bound(bmv, ymv, bb, rr))
            assert r["ok"], (fmt, N, K, batch, case, r)


@pytest.mark.parametrize("fmt", wl.FORMATS)
@pytest.mark.parametrize("batch", [1, 2, 8, 9, 11])
def test_swiglu(qmv, fmt, batch):
    for N, K in SHAPES:
        if K % wl.BLOCK[fmt]:
            continue
        xd = XDT.get(fmt, "f32")
        wg = wl.gen_weights(fmt, N, K, (62, N, K))
        wu = wl.gen_weights(fmt, N, K, (63, N, K))
        x = wl.gen_x(K, batch, xd, (62, N, K))
        _say("swiglu", fmt, N, K, batch)
        h = qmv.matvec_swiglu(fmt, pack_dev(qmv, fmt, wg), pack_dev(qmv, fmt, wu), dev_x(x, xd), N, K)
        torch.cuda.synchronize()
        g, dg = _prod(fmt, wg, x, xd)
        u, du = _prod(fmt, wu, x, xd)
        r = oracle.check_within(h.cpu().numpy(), oracle.swiglu_ref(g, u), oracle.swiglu_bound(g, u, dg, du))
        assert r["ok"], (fmt, N, K, batch, r)


@pytest.mark.parametrize("batch", [1, 8])
def test_swiglu_decoder_mlp_shape_and_graph(qmv, batch):
    # the 1.1B decoder's gate / up (5632 x 2048, Q4K), fused, captured in a
    # graph; at batch 8 on the matrix cores, several row tiles per workgroup
    fmt, N, K = "q4k", 5632, 2048
    wg = wl.gen_weights(fmt, N, K, (64, 0, 4))
    wu = wl.gen_weights(fmt, N, K, (64, 0, 5))
    x = wl.gen_x(K, batch, "f32", (64, 0, 4))
    Wg, Wu, xd = pack_dev(qmv, fmt, wg), pack_dev(qmv, fmt, wu), dev_x(x, "f32")
    h = torch.empty((batch, N), dtype=torch.float32, device="cuda")
    qmv.matvec_swiglu(fmt, Wg, Wu, xd, N, K, h=h)
    torch.cuda.synchronize()
    eager = h.clone()
    g, dg = _prod(fmt, wg, x, "f32")
    u, du = _prod(fmt, wu, x, "f32")
    r = oracle.check_within(eager.cpu().numpy(), oracle.swiglu_ref(g, u), oracle.swiglu_bound(g, u, dg, du))
    assert r["ok"], r
    s = torch.cuda.Stream()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=s):
        qmv.matvec_swiglu(fmt, Wg, Wu, xd, N, K, h=h)
    for _ in range(3):
        h.zero_()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(h.view(torch.int32), eager.view(torch.int32))


def test_epilogue_plain_equals_matvec_bitwise(qmv):
    # no bias, no residual: the same kernel and the same bits as qmv_matvec
    for fmt, N, K, b in (("q4k", 300, 2048, 1), ("q6k", 129, 5632, 1), ("q4k", 300, 2048, 8)):
        w = wl.gen_weights(fmt, N, K, (65, N, K))
        x = dev_x(wl.gen_x(K, b, "f32", (65, N, K)), "f32")
        Wp = pack_dev(qmv, fmt, w)
        a = qmv.matvec(fmt, Wp, x, N, K)
        c = qmv.matvec_ex(fmt, Wp, x, N, K)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int32), c.view(torch.int32)), (fmt, N, K, b)


@pytest.mark.parametrize("batch", [1, 8])
def test_fused_sweep_launch_configuration(qmv, batch):
    # the timed fused decode token's own launches for one 1.1B layer plus the
    # head: q + k + v grouped, o with the residual added in place, gate / up /
    # SwiGLU in one launch writing h, down reading h with the residual added in
    # place; every output against the oracle, the residual chain included
    import bench
    st = bench.FusedSweep(qmv, wl.c5_sweep(batch, layers=1), batch)
    r0 = st.resid.cpu().numpy().astype(np.float64)
    lay = st.layers[0]
    xin = {k: lay[k].cpu().numpy().astype(np.float64) for k in ("attn_in", "o_in", "mlp_in")}
    st()
    torch.cuda.synchronize()
    # one weight set per distinct shape (later matrices of that shape get
    # copies of it), seeded with the key of the shape's first matrix
    shapes = {nm: (fmt, N, K) for nm, fmt, N, K in wl.C5_LAYER}
    first = {}
    for i, (nm, fmt, N, K) in enumerate(wl.C5_LAYER):
        first.setdefault((fmt, N, K), (5, 0, i))
    keys = {nm: first[shapes[nm]] for nm in shapes}

    def prod(nm, x):
        fmt, N, K = shapes[nm]
        W32 = oracle.dequant(fmt, wl.gen_weights(fmt, N, K, keys[nm]))
        return oracle.matvec_ref(W32, x), oracle.tolerance_bound(W32, x, TAU)

    for nm in ("q", "k", "v"):
        y, b = prod(nm, xin["attn_in"])
        r = oracle.check_within(lay[nm].cpu().numpy(), y, b)
        _say("fused sweep", batch, nm, r)
        assert r["ok"], (nm, r)
    yo, bo = prod("o", xin["o_in"])
    r1 = oracle.epilogue_ref(yo, None, r0)
    b1 = oracle.epilogue_bound(bo, yo, None, r0)
    g, dg = prod("gate", xin["mlp_in"])
    u, du = prod("up", xin["mlp_in"])
    h = lay["h"].cpu().numpy()
    r = oracle.check_within(h, oracle.swiglu_ref(g, u), oracle.swiglu_bound(g, u, dg, du))
    _say("fused sweep", batch, "swiglu", r)
    assert r["ok"], r
    # down reads the kernel's own h (its error is checked above); the residual
    # it adds to carries the o step's bound
    yd, bd = prod("down", h.astype(np.float64))
    r2 = oracle.epilogue_ref(yd, None, r1)
    b2 = oracle.epilogue_bound(bd, yd, None, r1) + b1
    r = oracle.check_within(st.resid.cpu().numpy(), r2, b2)
    _say("fused sweep", batch, "residual chain", r)
    assert r["ok"], r
    Wh, xh, yh, V = st.head
    W32 = oracle.dequant("q6k", wl.gen_weights("q6k", V, 2048, (5, 1000, 7)))
    xv = xh.cpu().numpy().astype(np.float64)
    r = oracle.check_within(yh.cpu().numpy(), oracle.matvec_ref(W32, xv), oracle.tolerance_bound(W32, xv, TAU))
    _say("fused sweep", batch, "head", r)
    assert r["ok"], r


@pytest.mark.parametrize("fmt,N,K", [("q6k", 2048, 5632), ("q4k", 2048, 2048), ("w4a16_g64", 2048, 5632),
                                     ("q8_0", 1, 64), ("q4k", 17, 256), ("q5_0", 1, 32)])
@pytest.mark.parametrize("batch", [1, 8])
def test_residual_epilogue_sizes(qmv, fmt, N, K, batch):
    # the decoder's o / down shapes with the residual added in place, and the
    # smallest and ragged shapes (one row, 17 rows, one block of K)
    xd = XDT.get(fmt, "f32")
    w = wl.gen_weights(fmt, N, K, (66, N, K))
    x = wl.gen_x(K, batch, xd, (66, N, K))
    res = np.random.default_rng(N + K).normal(0, 2, (batch, N)).astype(np.float32)
    rd = dev(res)
    qmv.matvec_ex(fmt, pack_dev(qmv, fmt, w), dev_x(x, xd), N, K, y=rd, residual=rd)
    torch.cuda.synchronize()
    y, b = _prod(fmt, w, x, xd)
    r = oracle.check_within(rd.cpu().numpy(), oracle.epilogue_ref(y, None, res), oracle.epilogue_bound(b, y, None, res))
    _say("residual", fmt, N, K, batch, r)
    assert r["ok"], r
