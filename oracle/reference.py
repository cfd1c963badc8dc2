"""f64 reference products and the tolerance bound (oracle; test infrastructure).

The method computes y = W x (decode, a batch of b vectors) and Y = X W^T
(prefill) directly from the packed blocks; its plain definition is the same
product over the dequantized f32 matrix W.  Here every weight and activation
is widened to float64 (exact) and the products are summed in float64, so the
only error of the reference is the f64 summation, about K * 2^-53 relative.
(aot-llm README, Metal backend notes: GPU kernels with f32 activations land
about 1e-6 relative to an f64 reference; pytensor-ml issue 53, PR 16: packed
matmul ops checked against an independently produced reference.)

Tolerance, per output element (b, n):

    |y[b][n] - y_ref[b][n]| <= tau * ||W[n, :]||_2 * ||x[b, :]||_2

with Euclidean norms over the dequantized f32 row and the activation vector
actually passed, both computed in f64.  tau = 1e-3 for outputs accumulated in
f32, 2e-2 for outputs of the bf16 matrix-core GEMM (bf16-rounded weights and
a bf16-rounded result).
"""
from __future__ import annotations

import numpy as np

TAU_F32 = 1e-3
TAU_BF16 = 2e-2


def matvec_ref(w32: np.ndarray, x) -> np.ndarray:
    """y[b][n] = sum_k w[n][k] * x[b][k] in float64.  x: [b][K] (or [K]); returns [b][N]."""
    x64 = np.atleast_2d(np.asarray(x, dtype=np.float64))
    return x64 @ np.asarray(w32, dtype=np.float64).T


def gemm_ref(w32: np.ndarray, X) -> np.ndarray:
    """Y[m][n] = sum_k X[m][k] * w[n][k] in float64 (same product, M rows)."""
    return matvec_ref(w32, X)


def tolerance_bound(w32: np.ndarray, x, tau: float) -> np.ndarray:
    """tau * ||W_row||_2 * ||x_b||_2 for every output, shape [b][N]."""
    x64 = np.atleast_2d(np.asarray(x, dtype=np.float64))
    wn = np.sqrt(np.sum(np.asarray(w32, dtype=np.float64) ** 2, axis=1))
    xn = np.sqrt(np.sum(x64 ** 2, axis=1))
    return tau * xn[:, None] * wn[None, :]


def check_within(y, y_ref, bound) -> dict:
    """Compare outputs against the reference; returns summary statistics.

    `ok` is True when every |y - y_ref| <= bound (and y is finite).
    `max_norm_err` is max |y - y_ref| / (bound / tau) style ratio: the error
    divided by the bound (<= 1 passes).
    """
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    err = np.abs(y - y_ref)
    finite = bool(np.all(np.isfinite(y)))
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / bound, np.where(err == 0, 0.0, np.inf))
    return {
        "ok": finite and bool(np.all(err <= bound)),
        "max_ratio": float(np.max(ratio)) if ratio.size else 0.0,
        "max_abs": float(np.max(err)) if err.size else 0.0,
        "n_exact_f32": int(np.sum(y.astype(np.float32) == y_ref.astype(np.float32))),
        "n": int(y.size),
    }
