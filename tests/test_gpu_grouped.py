"""GPU parity of the grouped matvec (several matrices of one K per call, one
format or several) against the CPU oracle, and against one qmv_matvec call
per matrix.

Bar: every output within 1e-3 * ||W_row|| * ||x|| of the f64 oracle; with
the same inputs the grouped call returns exactly what the single calls
return (each row is summed in the same order whichever matrix it belongs to;
the one exception, batch 1 with 512 < K <= 1024 across 16384 rows, is not
among these shapes).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_helpers import check_every_row, TAU, dev_x, pack_dev, x_values

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _make(qmv, fmt, shapes, K, batch, x_dtype, shared_x, seed):
    """Seeded matrices of the given row counts, packed, plus their activations."""
    ws, Wps, xs = [], [], []
    x0 = wl.gen_x(K, batch, x_dtype, (30, seed, 0))
    for i, N in enumerate(shapes):
        w = wl.gen_weights(fmt, N, K, (30, seed, i + 1))
        ws.append(w)
        Wps.append(pack_dev(qmv, fmt, w))
        xs.append(x0 if shared_x else wl.gen_x(K, batch, x_dtype, (30, seed, 100 + i)))
    return ws, Wps, xs


def _run_and_check(qmv, fmt, shapes, K, batch, x_dtype, shared_x, seed, rows_cap=None):
    ws, Wps, xs = _make(qmv, fmt, shapes, K, batch, x_dtype, shared_x, seed)
    xd = {}
    items = []
    for i, (Wp, x) in enumerate(zip(Wps, xs)):
        key = id(x)
        if key not in xd:
            xd[key] = dev_x(x, x_dtype)
        items.append((Wp, xd[key], shapes[i]))
    ys = qmv.matvec_grouped(fmt, items, K)
    torch.cuda.synchronize()
    for i, (w, x, y) in enumerate(zip(ws, xs, ys)):
        N = shapes[i]
        rows = np.arange(N)
        if rows_cap is not None and N > rows_cap:
            g = np.random.default_rng(i)
            rows = np.unique(np.concatenate([[0, N - 1], g.integers(0, N, rows_cap)]))
        W32 = oracle.dequant_rows(fmt, w, rows)
        xv = x_values(x, x_dtype)
        ref = oracle.matvec_ref(W32, xv)
        bound = oracle.tolerance_bound(W32, xv, TAU["matvec"])
        r = oracle.check_within(y.cpu().numpy()[:, rows], ref, bound)
        assert r["ok"], (fmt, i, N, r)
    return ws, Wps, xd, items, ys


XDT = {"q8_0": "f32", "w4a16_g64": "f16", "q4k": "f32", "q6k": "f32", "q4_0": "f32", "q5_0": "f32", "q5k": "f32",
       "bf16": "f32", "i8row": "f32"}


@pytest.mark.parametrize("fmt", wl.FORMATS)
@pytest.mark.parametrize("shared_x", [True, False])
def test_grouped_parity_ragged(qmv, fmt, shared_x):
    K = wl.BLOCK[fmt] * 8
    shapes = [1, 67, 300, 5, 129]
    _say(fmt, shared_x, shapes, K)
    _run_and_check(qmv, fmt, shapes, K, 1, XDT[fmt], shared_x, seed=1)


def test_grouped_w4a16_f32_activations(qmv):
    _run_and_check(qmv, "w4a16_g64", [640, 64, 3], 2048, 1, "f32", False, seed=2)


@pytest.mark.parametrize("fmt", ["q4k", "w4a16_g64"])
def test_grouped_more_items_than_one_launch_holds(qmv, fmt):
    # 37 items: three launches of up to 16; x shared in runs of three
    K = wl.BLOCK[fmt] * 4
    shapes = [int(n) for n in np.random.default_rng(3).integers(1, 200, 37)]
    ws, Wps, xs = _make(qmv, fmt, shapes, K, 1, XDT[fmt], False, seed=3)
    xdev = [dev_x(xs[i - i % 3], XDT[fmt]) for i in range(len(shapes))]
    ys = qmv.matvec_grouped(fmt, [(Wps[i], xdev[i], shapes[i]) for i in range(len(shapes))], K)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        W32 = oracle.dequant_rows(fmt, ws[i], np.arange(shapes[i]))
        xv = x_values(xs[i - i % 3], XDT[fmt])
        r = oracle.check_within(ys[i].cpu().numpy(), oracle.matvec_ref(W32, xv),
                                oracle.tolerance_bound(W32, xv, TAU["matvec"]))
        assert r["ok"], (i, r)


@pytest.mark.parametrize("fmt", wl.FORMATS)
def test_grouped_equals_single_calls_bitwise(qmv, fmt):
    K = wl.BLOCK[fmt] * 16
    shapes = [700, 64, 2049]
    ws, Wps, xd, items, ys = _run_and_check(qmv, fmt, shapes, K, 1, XDT[fmt], True, seed=4)
    for (Wp, x, N), y in zip(items, ys):
        single = qmv.matvec(fmt, Wp, x, N, K)
        torch.cuda.synchronize()
        assert torch.equal(single.view(torch.int32), y.view(torch.int32))


@pytest.mark.parametrize("fmt", wl.FORMATS)
@pytest.mark.parametrize("batch", [2, 8, 11])
@pytest.mark.parametrize("shared_x", [True, False])
def test_grouped_batched_parity(qmv, fmt, batch, shared_x):
    # batch >= 2: the matrix-core kernel, items laid side by side (11: two chunks)
    K = wl.BLOCK[fmt] * 8
    _run_and_check(qmv, fmt, [300, 17, 1, 129], K, batch, XDT[fmt], shared_x, seed=5)


def test_grouped_batched_many_items_and_wide_k(qmv):
    shapes = [int(n) for n in np.random.default_rng(8).integers(1, 90, 19)]
    _run_and_check(qmv, "q6k", shapes, 2048, 8, "f32", False, seed=8)
    # K past the matrix-core kernel's range: one launch per item
    _run_and_check(qmv, "q4k", [40, 9], 6400, 8, "f32", True, seed=9)


@pytest.mark.parametrize("fmt", ["q4k", "q6k", "w4a16_g64"])
def test_grouped_batched_equals_single_calls_bitwise(qmv, fmt):
    K = wl.BLOCK[fmt] * 16 if fmt != "w4a16_g64" else 4096
    shapes = [700, 64, 2049]
    ws, Wps, xd, items, ys = _run_and_check(qmv, fmt, shapes, K, 8, XDT[fmt], True, seed=10)
    for (Wp, x, N), y in zip(items, ys):
        single = qmv.matvec(fmt, Wp, x, N, K)
        torch.cuda.synchronize()
        assert torch.equal(single.view(torch.int32), y.view(torch.int32))


@pytest.mark.parametrize("fmt", wl.FORMATS)
@pytest.mark.parametrize("batch", [3, 8])
def test_grouped_batched_several_tiles_per_workgroup(qmv, fmt, batch):
    # 1066 tiles of 16 rows at K = 2048 against at most 256 workgroups (512
    # for Q6K): workgroups take two to five tiles each, ragged per segment,
    # the 8-block kernels taking them with two staging register sets in turn.
    # Rows sampled for the oracle; the single calls (another split of the
    # tiles over workgroups) must return the same bits.
    K = 2048
    shapes = [5000, 3001, 17, 9000]
    _say(fmt, batch, shapes)
    ws, Wps, xd, items, ys = _run_and_check(qmv, fmt, shapes, K, batch, XDT[fmt], False, seed=12, rows_cap=1500)
    for (Wp, x, N), y in zip(items, ys):
        single = qmv.matvec(fmt, Wp, x, N, K)
        torch.cuda.synchronize()
        assert torch.equal(single.view(torch.int32), y.view(torch.int32)), (fmt, N)


def test_grouped_wide_k_falls_back(qmv):
    # K = 16384 with f32 activations needs more activation registers than the
    # grouped single-vector kernel holds: one launch per item instead
    _run_and_check(qmv, "q8_0", [40, 9], 16384, 1, "f32", False, seed=6)


def test_grouped_graph_replay(qmv):
    fmt, K = "q4k", 2048
    shapes = [2048, 256, 5632]
    ws, Wps, xs = _make(qmv, fmt, shapes, K, 1, "f32", True, seed=7)
    x = dev_x(xs[0], "f32")
    items = [(Wps[i], x, shapes[i]) for i in range(3)]
    eager = [y.clone() for y in qmv.matvec_grouped(fmt, items, K)]
    outs = [torch.empty_like(e) for e in eager]
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        qmv.matvec_grouped(fmt, [it + (o,) for it, o in zip(items, outs)], K)
    for _ in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e)


def test_config_w4a16_gate_up_grouped(qmv):
    # the 1.1B MLP's gate and up projections share x: one grouped call
    c = wl.c2_w4a16_mlp()
    (_, fmt, N, K, kg), (_, _, _, _, ku) = c["mats"][0], c["mats"][1]
    wg, wu = wl.gen_weights(fmt, N, K, kg), wl.gen_weights(fmt, N, K, ku)
    x = wl.gen_x(K, 1, "f16", kg)
    xt = dev_x(x, "f16")
    yg, yu = qmv.matvec_grouped(fmt, [(pack_dev(qmv, fmt, wg), xt, N), (pack_dev(qmv, fmt, wu), xt, N)], K)
    torch.cuda.synchronize()
    xv = x_values(x, "f16")
    for w, y in ((wg, yg), (wu, yu)):
        W32 = oracle.dequant_rows(fmt, w, np.arange(N))
        r = oracle.check_within(y.cpu().numpy(), oracle.matvec_ref(W32, xv),
                                oracle.tolerance_bound(W32, xv, TAU["matvec"]))
        _say(r)
        assert r["ok"], r


@pytest.mark.parametrize("batch", [1, 8])
def test_config_decode_layer_qkv_grouped(qmv, batch):
    # q and k (Q4K) and v (Q6K) of one 1.1B decoder layer in one mixed call;
    # each output equals its own single call bit for bit
    layer = [m for m in wl.c5_sweep(1, layers=1)["mats"] if m[0] in ("l0.q", "l0.k", "l0.v")]
    x = wl.gen_x(2048, batch, "f32", (31, 0, 0))
    xt = dev_x(x, "f32")
    xv = x_values(x, "f32")
    ws = {nm: wl.gen_weights(fmt, N, K, key) for nm, fmt, N, K, key in layer}
    Wp = {nm: pack_dev(qmv, fmt, ws[nm]) for nm, fmt, N, K, key in layer}
    ys = qmv.matvec_grouped(None, [(Wp[nm], xt, N, None, fmt) for nm, fmt, N, K, key in layer], 2048)
    torch.cuda.synchronize()
    for (nm, fmt, N, K, key), y in zip(layer, ys):
        W32 = oracle.dequant_rows(fmt, ws[nm], np.arange(N))
        r = oracle.check_within(y.cpu().numpy(), oracle.matvec_ref(W32, xv),
                                oracle.tolerance_bound(W32, xv, TAU["matvec"]))
        _say(nm, batch, r)
        assert r["ok"], (nm, r)
        single = qmv.matvec(fmt, Wp[nm], xt, N, K)
        torch.cuda.synchronize()
        assert torch.equal(single.view(torch.int32), y.view(torch.int32)), nm


@pytest.mark.parametrize("batch", [1, 3, 8, 11])
def test_grouped_mixed_kquant_ragged(qmv, batch):
    # Q4K and Q6K items interleaved in one call (one launch per 16 items and
    # chunk of 8 vectors), ragged rows, K over several super-blocks
    K = 256 * 6
    fmts = ["q4k", "q6k", "q6k", "q4k", "q6k"] * 4  # 20 items: two launches at batch 1
    shapes = [int(n) for n in np.random.default_rng(12).integers(1, 180, len(fmts))]
    x = wl.gen_x(K, batch, "f32", (32, batch, 0))
    xt = dev_x(x, "f32")
    xv = x_values(x, "f32")
    ws = [wl.gen_weights(f, n, K, (32, batch, i + 1)) for i, (f, n) in enumerate(zip(fmts, shapes))]
    Wp = [pack_dev(qmv, f, w) for f, w in zip(fmts, ws)]
    ys = qmv.matvec_grouped("q4k", [(Wp[i], xt, shapes[i], None, None if fmts[i] == "q4k" else "q6k")
                                    for i in range(len(fmts))], K)
    torch.cuda.synchronize()
    _say(batch, shapes)
    for i, (f, n, w, y) in enumerate(zip(fmts, shapes, ws, ys)):
        W32 = oracle.dequant_rows(f, w, np.arange(n))
        r = oracle.check_within(y.cpu().numpy(), oracle.matvec_ref(W32, xv),
                                oracle.tolerance_bound(W32, xv, TAU["matvec"]))
        assert r["ok"], (i, f, n, r)
        single = qmv.matvec(f, Wp[i], xt, n, K)
        torch.cuda.synchronize()
        assert torch.equal(single.view(torch.int32), y.view(torch.int32)), (i, f, n)


@pytest.mark.parametrize("batch", [1, 8])
def test_grouped_mixed_outside_kernel_range_falls_back(qmv, batch):
    # Q4K / Q6K mix at K = 6400: past the batched kernel's K and the single-vector
    # kernel's register budget for f32 activations, so one launch per item
    K = 6400
    fmts, shapes = ["q4k", "q6k", "q4k"], [40, 9, 130]
    x = wl.gen_x(K, batch, "f32", (34, batch, 0))
    xt = dev_x(x, "f32")
    xv = x_values(x, "f32")
    ws = [wl.gen_weights(f, n, K, (34, batch, i + 1)) for i, (f, n) in enumerate(zip(fmts, shapes))]
    Wp = [pack_dev(qmv, f, w) for f, w in zip(fmts, ws)]
    ys = qmv.matvec_grouped(None, [(Wp[i], xt, shapes[i], None, fmts[i]) for i in range(3)], K)
    torch.cuda.synchronize()
    for i, (f, n, w, y) in enumerate(zip(fmts, shapes, ws, ys)):
        W32 = oracle.dequant_rows(f, w, np.arange(n))
        r = oracle.check_within(y.cpu().numpy(), oracle.matvec_ref(W32, xv),
                                oracle.tolerance_bound(W32, xv, TAU["matvec"]))
        assert r["ok"], (i, f, n, r)


@pytest.mark.parametrize("batch", [1, 8])
def test_grouped_mixed_other_formats_split(qmv, batch):
    # Q8_0, W4A16 (f32 activations) and Q4K in one call: one launch series per
    # format, results as their single calls
    K = 2048
    fmts = ["q8_0", "w4a16_g64", "q4k", "q8_0", "w4a16_g64"]
    shapes = [100, 257, 64, 3, 1000]
    x = wl.gen_x(K, batch, "f32", (33, batch, 0))
    xt = dev_x(x, "f32")
    xv = x_values(x, "f32")
    ws = [wl.gen_weights(f, n, K, (33, batch, i + 1)) for i, (f, n) in enumerate(zip(fmts, shapes))]
    Wp = [pack_dev(qmv, f, w) for f, w in zip(fmts, ws)]
    ys = qmv.matvec_grouped(None, [(Wp[i], xt, shapes[i], None, fmts[i]) for i in range(len(fmts))], K)
    torch.cuda.synchronize()
    for i, (f, n, w, y) in enumerate(zip(fmts, shapes, ws, ys)):
        W32 = oracle.dequant_rows(f, w, np.arange(n))
        r = oracle.check_within(y.cpu().numpy(), oracle.matvec_ref(W32, xv),
                                oracle.tolerance_bound(W32, xv, TAU["matvec"]))
        assert r["ok"], (i, f, n, r)
        single = qmv.matvec(f, Wp[i], xt, n, K)
        torch.cuda.synchronize()
        assert torch.equal(single.view(torch.int32), y.view(torch.int32)), (i, f, n)


@pytest.mark.parametrize("batch", [1, 8])
def test_decode_sweep_launch_configuration(qmv, batch):
    # the timed decode sweep's own launches (q + k and gate + up grouped), one
    # 1.1B decoder layer plus the 32000-row head, against the oracle
    import bench
    cfg = wl.c5_sweep(batch, layers=1)
    st = bench.Sweep(qmv, cfg, batch)
    st()
    torch.cuda.synchronize()
    # weights and activations as the sweep draws them: one weight set per
    # distinct shape (later matrices of that shape get copies of it), one vector
    # set per shared input, each seeded with the key of the first matrix
    first_key, shape_key = {}, {}
    outs = [it[3] for _, _, items in st.calls for it in items]
    assert len(outs) == len(cfg["mats"])
    for (name, fmt, N, K, key), y in zip(cfg["mats"], outs):
        layer, nm = name.split(".") if "." in name else ("", name)
        share = (layer, bench.Sweep.SHARED.get(nm, nm))
        first_key.setdefault(share, key)
        shape_key.setdefault((fmt, N, K), key)
        x = wl.gen_x(K, batch, "f32", first_key[share])
        w = wl.gen_weights(fmt, N, K, shape_key[(fmt, N, K)])
        r = check_every_row(fmt, w, y.cpu().numpy(), x.astype(np.float64))  # every row, head included
        _say(name, batch, r)
        assert r["ok"], (name, batch, r)


@pytest.mark.parametrize("fmt,shapes", [("q4k", [5632, 5632]), ("q6k", [5000, 4000, 100]), ("q8_0", [8300])])
def test_grouped_f32_four_row_groups(qmv, fmt, shapes):
    """K = 2048 with f32 activations and 8193..16384 rows in one launch: the
    launch takes four rows per lane group (every wave then has one row group),
    where each matrix on its own (at most 8192 rows) takes two.  Sampled rows
    match the oracle, and the grouped call equals the single calls bit for bit
    (a row's lanes are folded in the same order for one, two or four rows)."""
    K = 2048
    ws, Wps, xd, items, ys = _run_and_check(qmv, fmt, shapes, K, 1, "f32", True, seed=23, rows_cap=512)
    for i, (Wp, x, N) in enumerate(items):
        y1 = qmv.matvec(fmt, Wp, x, N, K)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int32), ys[i].view(torch.int32)), (fmt, i, N)
