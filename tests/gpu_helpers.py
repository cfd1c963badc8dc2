"""Shared helpers for the GPU tests: upload seeded logical arrays, pack them
with the HIP library and compare against the CPU oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads as wl

TAU = {"matvec": oracle.reference.TAU_F32, "gemm": oracle.reference.TAU_BF16}


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def dev_x(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Activations to the device: f32 values, or f16 / bf16 bit patterns."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
    return t.view(torch.float16 if dtype == "f16" else torch.bfloat16)


def x_values(x: np.ndarray, dtype: str) -> np.ndarray:
    """The activation values the kernel sees, exactly, as float64."""
    if dtype == "f32":
        return x.astype(np.float64)
    return oracle.f16_to_f64(x) if dtype == "f16" else oracle.bf16_to_f64(x)


def pack_dev(qmv, fmt: str, w: dict) -> torch.Tensor:
    d = {k: dev(v) for k, v in w.items()}
    return qmv.pack(fmt, d)


def check_matvec(qmv, fmt, w, x, x_dtype, rows=None, tau=None):
    """Run the HIP matvec on packed w and compare (optionally sampled rows) with the oracle."""
    N, K = w["q"].shape
    Wp = pack_dev(qmv, fmt, w)
    y = qmv.matvec(fmt, Wp, dev_x(x, x_dtype), N, K)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    rows = np.arange(N) if rows is None else np.asarray(rows)
    W32 = oracle.dequant_rows(fmt, w, rows)
    xv = x_values(x, x_dtype)
    ref = oracle.matvec_ref(W32, xv)
    bound = oracle.tolerance_bound(W32, xv, tau or TAU["matvec"])
    return oracle.check_within(y[:, rows], ref, bound), y, ref


def check_every_row(fmt, w, y, xv, tau=None, chunk=8192):
    """Compare every output row of y [b][N] with the oracle, dequantizing the
    matrix in chunks of rows (vocab heads would not fit as one f64 block)."""
    N = w["q"].shape[0]
    worst = {"ok": True, "max_ratio": 0.0, "rows": N}
    for r0 in range(0, N, chunk):
        rows = np.arange(r0, min(N, r0 + chunk))
        W32 = oracle.dequant_rows(fmt, w, rows)
        r = oracle.check_within(y[:, rows], oracle.matvec_ref(W32, xv),
                                oracle.tolerance_bound(W32, xv, tau or TAU["matvec"]))
        worst["ok"] = worst["ok"] and r["ok"]
        worst["max_ratio"] = max(worst["max_ratio"], r["max_ratio"])
        if not r["ok"]:
            worst["first_bad_chunk"] = (r0, r)
            break
    return worst
