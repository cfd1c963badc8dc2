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


# ----------------------------------------------------------------------------
# Fused decode epilogues (aot-llm README, Metal backend notes: the q/k/v
# projections take their biases in the epilogue of the matrix kernels, wo and
# down add the residual in theirs, and gate / up / SwiGLU run as one fused
# product).  The plain definitions, in f64:
#
#   epilogue:  y[b][n] = residual[b][n] + ((W x_b)[n] + bias[n])
#   SwiGLU:    h[b][n] = silu((W_gate x_b)[n]) * (W_up x_b)[n],
#              silu(z) = z / (1 + exp(-z))   (the swish with unit slope)
#
# Tolerance.  The products carry the matvec bound d = tau ||W_row|| ||x||.
# The epilogue adds at most two f32 roundings of the result on top:
#   |y - y*| <= d + 2^-23 (|residual| + |W x + bias|) + 2^-24 |bias|.
# For SwiGLU, with g*, u* the exact products and dg, du their bounds:
#   |silu(g) u - silu(g*) u*| <= L dg (|u*| + du) + |silu(g*)| du
# where L = 1.1 >= max |silu'| = 1.09984 (silu' = s (1 + z (1 - s)), s the
# logistic function, peaks near z = 2.40), plus the f32 evaluation of silu and the
# product, allowed 2^-20 |h*| (a few ulp of each step).

SILU_LIP = 1.1


def silu_ref(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu_ref(g, u):
    """h = silu(g) * u, elementwise, in f64."""
    return silu_ref(g) * np.asarray(u, dtype=np.float64)


def swiglu_bound(g_ref, u_ref, dg, du):
    """Bound on |h - h*| from the bounds dg, du of the two products (shapes broadcast)."""
    g_ref = np.asarray(g_ref, dtype=np.float64)
    u_ref = np.asarray(u_ref, dtype=np.float64)
    h = np.abs(swiglu_ref(g_ref, u_ref))
    return SILU_LIP * dg * (np.abs(u_ref) + du) + np.abs(silu_ref(g_ref)) * du + 2.0 ** -20 * h


def epilogue_ref(y_mv, bias=None, residual=None):
    """residual + (W x + bias) in f64; y_mv is the exact product [b][N]."""
    y = np.asarray(y_mv, dtype=np.float64)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    if residual is not None:
        y = np.asarray(residual, dtype=np.float64) + y
    return y


def epilogue_bound(bound_mv, y_mv, bias=None, residual=None):
    """The matvec bound plus the two f32 roundings of the epilogue."""
    y_mv = np.asarray(y_mv, dtype=np.float64)
    t = y_mv + (0.0 if bias is None else np.asarray(bias, dtype=np.float64)[None, :])
    r = 0.0 if residual is None else np.abs(np.asarray(residual, dtype=np.float64))
    b = 0.0 if bias is None else np.abs(np.asarray(bias, dtype=np.float64))[None, :]
    return bound_mv + 2.0 ** -23 * (r + np.abs(t)) + 2.0 ** -24 * b
