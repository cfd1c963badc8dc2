"""GPU parity of the W4A16 prefill GEMM (bf16 MFMA) against the CPU oracle.

Bar: every output within 2e-2 * ||W_row|| * ||X_row|| of the f64 product of
the exact f32 dequantized weights.  A second, diagnostic reference with the
weights rounded to bf16 (what the matrix cores consume) must agree far more
tightly: only the f32 summation order and the final bf16 rounding differ.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_helpers import dev, dev_x, pack_dev

pytestmark = pytest.mark.gpu

FMT = "w4a16_g64"


def _say(*a):
    print(*a, flush=True)


def _bf16_round(a32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a32)).to(torch.bfloat16).to(torch.float32)
    return t.numpy()


def run_gemm(qmv, N, K, M, key):
    w = wl.gen_weights(FMT, N, K, key)
    Xb = wl.gen_x(K, M, "bf16", key)
    Wp = pack_dev(qmv, FMT, w)
    Y = qmv.gemm(FMT, Wp, dev_x(Xb, "bf16"), N, K)
    torch.cuda.synchronize()
    return w, Xb, Y.float().cpu().numpy()


# Shapes reach every kernel configuration the dispatcher picks: M <= 16 (the K
# split for K <= 2048, one 16-token tile past it), M <= 32 (64 x 32 tiles of
# weight rows x tokens) and larger M (64 x 64), with ragged rows, tokens and K
# (K not a multiple of the 128-k step, K = 64), and the full 5632 x 2048
# matrix at M = 1 .. 512.  Every output is compared.
@pytest.mark.parametrize("N,K,M", [(40, 64, 1), (200, 640, 17), (130, 128, 33), (96, 256, 129),
                                   (200, 640, 5), (72, 1984, 16), (1000, 2048, 3), (24, 2176, 16),
                                   (2900, 704, 900), (4200, 320, 100), (1000, 1088, 300), (64, 2560, 40), (100, 64, 50),
                                   (5632, 2048, 1), (5632, 2048, 16), (5632, 2048, 17),
                                   (5632, 2048, 128), (5632, 2048, 512)])
def test_gemm_parity(qmv, N, K, M):
    _say("gemm", N, K, M)
    w, Xb, Y = run_gemm(qmv, N, K, M, (21, N, K))
    W32 = oracle.dequant(FMT, w)
    X = oracle.bf16_to_f64(Xb)
    rows = np.arange(N)  # every output is compared
    ref = oracle.gemm_ref(W32[rows], X)
    r = oracle.check_within(Y[:, rows], ref, oracle.tolerance_bound(W32[rows], X, 2e-2))
    _say(r)
    assert r["ok"], r
    # diagnostic: with bf16 weights the only differences are summation order and the output rounding
    ref_b = oracle.gemm_ref(_bf16_round(W32[rows]), X)
    rb = oracle.check_within(Y[:, rows], ref_b, oracle.tolerance_bound(W32[rows], X, 1e-2))
    assert rb["ok"] and rb["max_ratio"] < 0.5, rb


def test_gemm_one_row_matches_matvec(qmv):
    N, K = 5632, 2048
    w = wl.gen_weights(FMT, N, K, (22, 0, 0))
    Xb = wl.gen_x(K, 1, "bf16", (22, 0, 0))
    Wp = pack_dev(qmv, FMT, w)
    Y = qmv.gemm(FMT, Wp, dev_x(Xb, "bf16"), N, K).float().cpu().numpy()
    xf = torch.from_numpy(oracle.bf16_to_f32(Xb)).cuda()
    y = qmv.matvec(FMT, Wp, xf, N, K).cpu().numpy()
    W32 = oracle.dequant(FMT, w)
    bound = oracle.tolerance_bound(W32, oracle.bf16_to_f64(Xb), 2e-2)
    assert np.all(np.abs(Y - y) <= bound)


def test_gemm_deterministic_and_graph_replay(qmv):
    N, K, M = 5632, 2048, 128
    w = wl.gen_weights(FMT, N, K, (23, 0, 0))
    Wp = pack_dev(qmv, FMT, w)
    X = dev_x(wl.gen_x(K, M, "bf16", (23, 0, 0)), "bf16")
    a = qmv.gemm(FMT, Wp, X, N, K).clone()
    b = qmv.gemm(FMT, Wp, X, N, K)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    Y = torch.empty_like(a)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        qmv.gemm(FMT, Wp, X, N, K, Y=Y)
    for _ in range(3):
        Y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), a.view(torch.int16))


def test_gemm_rejects_other_formats(qmv):
    w = wl.gen_weights("q4k", 64, 256, (24, 0, 0))
    Wp = pack_dev(qmv, "q4k", w)
    X = dev_x(wl.gen_x(256, 16, "bf16", (24, 0, 0)), "bf16")
    with pytest.raises(qmv.QmvError, match="W4A16"):
        qmv.gemm("q4k", Wp, X, 64, 256)
