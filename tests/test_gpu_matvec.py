"""GPU parity of the HIP pack / dequant / matvec path against the CPU oracle.

Bar: packing and dequantization bit-exact; one-hot matvec bit-exact (the
dequantized column); every matvec output within 1e-3 * ||W_row|| * ||x||.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_helpers import check_every_row, check_matvec, dev, dev_x, pack_dev, x_values

pytestmark = pytest.mark.gpu

XDT = {"q8_0": ("f32",), "w4a16_g64": ("f16", "f32"), "q4k": ("f32",), "q6k": ("f32",), "q4_0": ("f32",),
       "q5_0": ("f32",), "q5k": ("f32",), "bf16": ("f32",), "i8row": ("f32",)}


def _say(*a):
    print(*a, flush=True)


# --------------------------------------------------------------- pack/dequant

@pytest.mark.parametrize("fmt", wl.FORMATS)
@pytest.mark.parametrize("N,mult", [(1, 1), (5, 3), (67, 2)])
def test_pack_bytes_equal_reference(qmv, fmt, N, mult):
    K = wl.BLOCK[fmt] * mult
    w = wl.gen_weights(fmt, N, K, (11, N, mult))
    _say("pack", fmt, N, K)
    got = pack_dev(qmv, fmt, w).cpu().numpy()
    want = oracle.pack_ref(fmt, w)
    # padding bytes between planes are unspecified; compare the planes only
    from oracle import layout
    for name, (off, nb) in layout.plane_offsets(fmt, N, K).items():
        assert np.array_equal(got[off:off + nb], want[off:off + nb]), name
    back = oracle.unpack_ref(fmt, N, K, got)
    for k in w:
        assert np.array_equal(back[k], w[k]), k


@pytest.mark.parametrize("fmt", wl.FORMATS)
def test_pack_stacked_batch(qmv, fmt):
    N, K, B = 9, wl.BLOCK[fmt] * 2, 3
    ws = [wl.gen_weights(fmt, N, K, (12, i, 0)) for i in range(B)]
    stacked = {k: np.stack([w[k] for w in ws]) for k in ws[0]}
    d = {k: dev(v) for k, v in stacked.items()}
    got = qmv.pack(fmt, d, N=N, K=K, batch=B).cpu().numpy()
    one = qmv.packed_bytes(fmt, N, K)
    from oracle import layout
    for i in range(B):
        want = oracle.pack_ref(fmt, ws[i])
        for name, (off, nb) in layout.plane_offsets(fmt, N, K).items():
            assert np.array_equal(got[i * one + off:i * one + off + nb], want[off:off + nb])


@pytest.mark.parametrize("fmt", wl.FORMATS)
@pytest.mark.parametrize("N,mult", [(3, 1), (130, 4)])
def test_dequant_bit_exact(qmv, fmt, N, mult):
    K = wl.BLOCK[fmt] * mult
    w = wl.gen_weights(fmt, N, K, (13, N, mult))
    _say("dequant", fmt, N, K)
    Wp = pack_dev(qmv, fmt, w)
    got = qmv.dequant(fmt, Wp, N, K).cpu().numpy()
    want = oracle.dequant(fmt, w)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_f16_scale_decode_exhaustive(qmv):
    """All 65536 fp16 patterns as Q8_0 scales with q = 1: w must be the scale itself."""
    N, K = 2048, 1024
    scale = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(N, K // 32)
    w = {"q": np.ones((N, K), np.int8), "scale": scale}
    Wp = pack_dev(qmv, "q8_0", w)
    got = qmv.dequant("q8_0", Wp, N, K).cpu().numpy()[:, ::32].ravel()
    want = oracle.f16_to_f32(scale.ravel())
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def test_q4k_range_edge_and_subnormal_scales(qmv):
    N, K = 4, 256
    w = wl.gen_weights("q4k", N, K, (14, 0, 0))
    w["d"][0, 0], w["dmin"][0, 0] = 0x6400, 0x0001
    w["sc"][0, :] = 63
    w["m"][0, :] = 1
    w["q"][0, :] = 15
    w["d"][1, 0], w["dmin"][1, 0] = 0x0001, 0x03FF  # subnormals
    Wp = pack_dev(qmv, "q4k", w)
    got = qmv.dequant("q4k", Wp, N, K).cpu().numpy()
    want = oracle.dequant("q4k", w)
    assert np.all(got[0] == np.float32(967680.0))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


# ---------------------------------------------------------------- matvec

SHAPES = {  # (N, K) spanning lanes-per-row 16 / 32 / 64, ragged passes and ragged N
    "q8_0": [(1, 32), (37, 512), (300, 1024), (129, 2560)],
    "w4a16_g64": [(1, 64), (37, 1024), (300, 2048), (129, 5632)],
    "q4k": [(1, 256), (37, 1024), (300, 3072), (129, 5632)],
    "q6k": [(1, 256), (37, 768), (300, 2048), (129, 5632)],
    "q4_0": [(1, 32), (37, 576), (300, 2048), (129, 5632)],
    "q5_0": [(1, 32), (37, 576), (300, 1024), (129, 5632)],
    "q5k": [(1, 256), (37, 768), (300, 2048), (129, 5632)],
    "bf16": [(1, 32), (37, 544), (300, 1024), (129, 3072)],
    "i8row": [(1, 32), (37, 512), (300, 1024), (129, 3072)],
}


@pytest.mark.parametrize("fmt", wl.FORMATS)
@pytest.mark.parametrize("batch", [1, 2, 3, 8, 9, 11])
def test_matvec_parity(qmv, fmt, batch):
    for N, K in SHAPES[fmt]:
        for xd in XDT[fmt]:
            w = wl.gen_weights(fmt, N, K, (15, N, K))
            x = wl.gen_x(K, batch, xd, (15, N, K))
            _say("matvec", fmt, N, K, batch, xd)
            r, _, _ = check_matvec(qmv, fmt, w, x, xd)
            assert r["ok"], (fmt, N, K, batch, xd, r)


# K cases of the batched (2..8 vector) matrix-core path: one wave, 8 waves of 8
# blocks, 24 blocks per wave with a ragged last wave (and, for W4A16 / Q8_0,
# a ragged last chunk), the largest K it takes, and a K past it (other kernel)
MFMA_K = {
    "q8_0": [32, 2048, 2080, 6144, 6176],
    "w4a16_g64": [64, 2048, 2112, 6144, 6208],
    "q4k": [256, 2048, 3328, 6144, 6400],
    "q6k": [256, 2048, 3328, 5632, 6400],
    # formats the matrix-core kernel does not take: the FMA kernel at 1..64 units
    "q4_0": [32, 544, 2048, 5632, 6176],
    "q5_0": [32, 544, 2048, 5632, 6176],
    "q5k": [256, 768, 2048, 5632, 6400],
    "bf16": [32, 544, 2048, 3072, 4128],
    "i8row": [32, 544, 2048, 3072, 4128],
}


@pytest.mark.parametrize("fmt", wl.FORMATS)
@pytest.mark.parametrize("kcase", range(5))
@pytest.mark.parametrize("batch", [2, 8])
def test_batched_matvec_k_ranges(qmv, fmt, kcase, batch):
    K = MFMA_K[fmt][kcase]
    N = 37 if K > 4096 else 133
    w = wl.gen_weights(fmt, N, K, (22, kcase, batch))
    for xd in XDT[fmt]:
        x = wl.gen_x(K, batch, xd, (22, kcase, batch))
        r, _, _ = check_matvec(qmv, fmt, w, x, xd)
        assert r["ok"], (fmt, K, batch, xd, r)


# More tiles than workgroups at K > 2048 (16 blocks of K per wave): workgroups
# take one or two tiles in turn, with one weight register set refilled across
# tiles, and the last wave of each tile holds one chunk (K = 2304: 72 blocks
# over 5 waves).  The matrix-core launch caps the grid at 256 workgroups (512
# for Q6K), so 263 / 513 tiles give some workgroups a second tile.
@pytest.mark.parametrize("fmt,N", [("q4k", 4200), ("q6k", 8208), ("q8_0", 4200), ("w4a16_g64", 4200)])
@pytest.mark.parametrize("batch", [3, 8])
def test_batched_more_tiles_than_workgroups(qmv, fmt, N, batch):
    K = 2304
    w = wl.gen_weights(fmt, N, K, (23, N, batch))
    for xd in XDT[fmt]:
        print("tiles", fmt, N, K, batch, xd, flush=True)
        x = wl.gen_x(K, batch, xd, (23, N, batch))
        Wp = pack_dev(qmv, fmt, w)
        y = qmv.matvec(fmt, Wp, dev_x(x, xd), N, K)
        torch.cuda.synchronize()
        r = check_every_row(fmt, w, y.cpu().numpy(), x_values(x, xd))
        assert r["ok"], (fmt, N, K, batch, xd, r)


# K cases of the single-vector kernel: one 32-weight unit per lane, K split
# over 2 waves with a ragged second slice, over 2 and 3 waves in full, the
# largest K with activations held in registers (4 waves for fp16 W4A16), and a
# K past it (another kernel)
B1_K = {
    "q8_0": [2048, 2080, 4096, 6144, 6176],
    "w4a16_g64": [2048, 2112, 4096, 5632, 8192, 8256],
    "q4k": [2048, 2304, 4096, 5632, 6144, 6400],
    "q6k": [2048, 2304, 4096, 5632, 6144, 6400],
    "q4_0": [2048, 2080, 4096, 5632, 6144, 6176],
    "q5_0": [2048, 2080, 4096, 5632, 6144, 6176],
    "q5k": [2048, 2304, 4096, 5632, 6144, 6400],
    "bf16": [2048, 2080, 4096, 5632, 6144, 6176],
    "i8row": [2048, 2080, 4096, 5632, 6144, 6176],
}


@pytest.mark.parametrize("fmt", wl.FORMATS)
@pytest.mark.parametrize("kcase", range(6))
def test_single_vector_k_ranges(qmv, fmt, kcase):
    if kcase >= len(B1_K[fmt]):
        pytest.skip("no such case for this format")
    K = B1_K[fmt][kcase]
    for N in (1, 133):
        w = wl.gen_weights(fmt, N, K, (23, kcase, N))
        for xd in XDT[fmt]:
            x = wl.gen_x(K, 1, xd, (23, kcase, N))
            _say("b1", fmt, N, K, xd)
            r, _, _ = check_matvec(qmv, fmt, w, x, xd)
            assert r["ok"], (fmt, N, K, xd, r)


NARROW_K = {"q8_0": [544, 1024], "w4a16_g64": [576, 1024], "q4k": [768, 1024], "q6k": [768, 1024],
            "q4_0": [544, 1024], "q5_0": [544, 1024], "q5k": [768, 1024], "bf16": [544, 1024],
            "i8row": [544, 1024]}


@pytest.mark.parametrize("fmt", wl.FORMATS)
def test_single_vector_streaming_narrow_k(qmv, fmt):
    # 512 < K <= 1024 on more than 16384 rows: 16 lanes per row with two
    # blocks of 32 each and one row per lane group (at K = 544 / 576 / 768 the
    # second block of some lanes lies past K).  Sampled rows against the
    # oracle; a one-hot x returns the dequantized column bit for bit.
    N = 16389
    for K in NARROW_K[fmt]:
        w = wl.gen_weights(fmt, N, K, (41, K, 0))
        rows = np.unique(np.concatenate([_sample_rows(N, seed=K), np.arange(N - 40, N)]))
        W32 = oracle.dequant_rows(fmt, w, rows)
        Wp = pack_dev(qmv, fmt, w)
        for xd in XDT[fmt]:
            _say("narrow K", fmt, N, K, xd)
            x = wl.gen_x(K, 1, xd, (41, K, 1))
            r, _, _ = check_matvec(qmv, fmt, w, x, xd, rows=rows)
            assert r["ok"], (fmt, K, xd, r)
            for k in (0, 33, K - 1):
                oh = np.zeros((1, K), np.float64)
                oh[0, k] = 1.0
                xb = oh.astype(np.float32) if xd == "f32" else wl.to_f16_bits(oh)
                y = qmv.matvec(fmt, Wp, dev_x(xb, xd), N, K).cpu().numpy()
                assert np.array_equal(y[0, rows], W32[:, k]), (fmt, K, xd, k)


@pytest.mark.parametrize("fmt", ["w4a16_g64", "q6k"])
def test_one_hot_through_k_split_bit_exact(qmv, fmt):
    # K = 5632 runs split over three waves: every column still comes back
    # exactly as the dequantized weight
    N, K = 40, 5632
    w = wl.gen_weights(fmt, N, K, (24, 0, 0))
    Wp = pack_dev(qmv, fmt, w)
    W32 = oracle.dequant(fmt, w)
    xd = XDT[fmt][0]
    for k in (0, 2047, 2048, 4095, 4096, K - 1):
        x = np.zeros((1, K), np.float64)
        x[0, k] = 1.0
        xb = x.astype(np.float32) if xd == "f32" else wl.to_f16_bits(x)
        y = qmv.matvec(fmt, Wp, dev_x(xb, xd), N, K).cpu().numpy()
        assert np.array_equal(y[0], W32[:, k]), (fmt, k)


@pytest.mark.parametrize("fmt", wl.FORMATS)
def test_one_hot_returns_dequantized_column_bit_exact(qmv, fmt):
    N, K = 70, wl.BLOCK[fmt] * 8 if fmt != "w4a16_g64" else 2048
    w = wl.gen_weights(fmt, N, K, (16, 0, 0))
    W32 = oracle.dequant(fmt, w)
    Wp = pack_dev(qmv, fmt, w)
    for xd in XDT[fmt]:
        ks = [0, 1, 17, 31, 32, 255, K - 1][:8]
        x = np.zeros((len(ks), K), np.float64)
        for i, k in enumerate(ks):
            x[i, k] = 1.0
        xb = x.astype(np.float32) if xd == "f32" else wl.to_f16_bits(x)
        y = qmv.matvec(fmt, Wp, dev_x(xb, xd), N, K).cpu().numpy()
        for i, k in enumerate(ks):
            assert np.array_equal(y[i], W32[:, k]), (fmt, xd, k)


@pytest.mark.parametrize("fmt", ["q4k", "q6k", "w4a16_g64", "q5k", "q8_0", "i8row"])
@pytest.mark.parametrize("batch", [1, 8])
def test_positive_near_constant_activations(qmv, fmt, batch):
    # all-positive, nearly equal activations (1 + 0.01 N(0,1), and the same times
    # 1000): the decode offsets (codes biased by 1024 or 128 and removed with
    # the sum of x) cancel the most here, at the decoder's longest K
    N, K = 300, 5632
    w = wl.gen_weights(fmt, N, K, (24, N, K))
    rng = np.random.default_rng(24 + batch)
    for scale in (1.0, 1000.0):
        x = (scale * (1.0 + 0.01 * rng.standard_normal((batch, K)))).astype(np.float32)
        r, _, _ = check_matvec(qmv, fmt, w, x, "f32")
        print("near-constant x", fmt, batch, scale, r["max_ratio"], flush=True)
        assert r["ok"], (fmt, batch, scale, r)


def test_q8_0_minus_128(qmv):
    N, K = 8, 64
    w = wl.gen_weights("q8_0", N, K, (17, 0, 0))
    w["q"][:, ::3] = -128
    x = wl.gen_x(K, 2, "f32", (17, 0, 0))
    r, _, _ = check_matvec(qmv, "q8_0", w, x, "f32")
    assert r["ok"], r


@pytest.mark.parametrize("fmt", wl.FORMATS)
def test_matvec_deterministic(qmv, fmt):
    N, K = 500, wl.BLOCK[fmt] * 8
    w = wl.gen_weights(fmt, N, K, (18, 0, 0))
    xd = XDT[fmt][0]
    x = dev_x(wl.gen_x(K, 4, xd, (18, 0, 0)), xd)
    Wp = pack_dev(qmv, fmt, w)
    a = qmv.matvec(fmt, Wp, x, N, K).cpu().numpy()
    b = qmv.matvec(fmt, Wp, x, N, K).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_graph_replay_matches_eager(qmv):
    fmt, N, K = "q4k", 3072, 1024
    w = wl.gen_weights(fmt, N, K, (19, 0, 0))
    Wp = pack_dev(qmv, fmt, w)
    x = dev_x(wl.gen_x(K, 1, "f32", (19, 0, 0)), "f32")
    eager = qmv.matvec(fmt, Wp, x, N, K).clone()
    y = torch.empty_like(eager)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        qmv.matvec(fmt, Wp, x, N, K, y=y)
    for _ in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager)


# ------------------------------------------------------- full workload shapes

def _sample_rows(N, n=384, seed=0):
    g = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, N - 1], g.integers(0, N, n)]))


def test_config_q8_0_512(qmv):
    c = wl.c1_q8_0()
    for name, fmt, N, K, key in c["mats"]:
        w = wl.gen_weights(fmt, N, K, key)
        x = wl.gen_x(K, c["batch"], c["x_dtype"], key)
        r, _, _ = check_matvec(qmv, fmt, w, x, c["x_dtype"])
        _say(name, r)
        assert r["ok"], r


def test_config_w4a16_mlp(qmv):
    c = wl.c2_w4a16_mlp()
    for name, fmt, N, K, key in c["mats"]:
        w = wl.gen_weights(fmt, N, K, key)
        x = wl.gen_x(K, c["batch"], c["x_dtype"], key)
        r, _, _ = check_matvec(qmv, fmt, w, x, c["x_dtype"])
        _say(name, r)
        assert r["ok"], r


def _run_every_row(qmv, fmt, w, x, xd):
    N, K = w["q"].shape
    y = qmv.matvec(fmt, pack_dev(qmv, fmt, w), dev_x(x, xd), N, K)
    torch.cuda.synchronize()
    return check_every_row(fmt, w, y.cpu().numpy(), x_values(x, xd))


def test_config_q4k_mlp_and_vocab_head(qmv):
    # every output, the 151936-row head included (oracle in row chunks)
    c = wl.c3_q4k_0b6()
    for name, fmt, N, K, key in c["mats"]:
        w = wl.gen_weights(fmt, N, K, key)
        x = wl.gen_x(K, c["batch"], c["x_dtype"], key)
        r = _run_every_row(qmv, fmt, w, x, c["x_dtype"])
        _say(name, r)
        assert r["ok"], r


@pytest.mark.parametrize("batch", [1, 8])
def test_config_decode_sweep_layer_and_head(qmv, batch):
    # every output of one layer's seven matvecs and the 32000-row Q6K head
    c = wl.c5_sweep(batch, layers=1)
    for name, fmt, N, K, key in c["mats"]:
        w = wl.gen_weights(fmt, N, K, key)
        x = wl.gen_x(K, batch, "f32", key)
        r = _run_every_row(qmv, fmt, w, x, "f32")
        _say(name, batch, r)
        assert r["ok"], (name, r)


def test_matvec_code_plane_past_2gib(qmv):
    """A Q8_0 matrix whose code plane is past 2 GiB (N * K = 2^31 + 48 K bytes).

    The batch-1 kernels address a plane with 32-bit offsets and reserve
    offsets from 2^31 up for "read nothing", so they hand such a matrix to the
    general kernel, as the matrix-core kernel does for batch 2.  Sampled rows
    (first, last, a random spread) at batch 1 and 2 and through a grouped call
    with a small matrix beside it match the oracle."""
    fmt, K = "q8_0", 4096
    N = (1 << 31) // K + 48
    w = wl.gen_weights(fmt, N, K, (0, 0, 9))
    Wp = pack_dev(qmv, fmt, w)
    rows = np.unique(np.concatenate([_sample_rows(N, 256, seed=3), np.arange(N - 64, N)]))
    W32 = oracle.dequant_rows(fmt, w, rows)
    del w
    for batch in (1, 2):
        x = wl.gen_x(K, batch, "f32", (0, 0, 9))
        y = qmv.matvec(fmt, Wp, dev_x(x, "f32"), N, K)
        torch.cuda.synchronize()
        xv = x_values(x, "f32")
        r = oracle.check_within(y.cpu().numpy()[:, rows], oracle.matvec_ref(W32, xv),
                                oracle.tolerance_bound(W32, xv, oracle.reference.TAU_F32))
        _say("q8_0 plane past 2 GiB", batch, r)
        assert r["ok"], (batch, r)
    # grouped, batch 1: the big matrix beside a small one sharing x
    ws = wl.gen_weights(fmt, 96, K, (0, 1, 9))
    Ws = pack_dev(qmv, fmt, ws)
    x = wl.gen_x(K, 1, "f32", (0, 0, 9))
    xd = dev_x(x, "f32")
    yb, ys = qmv.matvec_grouped(fmt, [(Wp, xd, N), (Ws, xd, 96)], K)
    torch.cuda.synchronize()
    xv = x_values(x, "f32")
    for y, W, rr in ((yb, W32, rows), (ys, oracle.dequant_rows(fmt, ws, np.arange(96)), np.arange(96))):
        r = oracle.check_within(y.cpu().numpy()[:, rr], oracle.matvec_ref(W, xv),
                                oracle.tolerance_bound(W, xv, oracle.reference.TAU_F32))
        assert r["ok"], r
