#!/usr/bin/env python3
"""Benchmark of the fused dequantize-and-multiply hot path on one MI355X.

Headline (one JSON line on stdout): decode matvec throughput in achieved GB/s
of algorithmic bytes, on the group-64 W4A16 MLP matvecs of a 1.1B-parameter
decoder (gate / up 5632 x 2048, down 2048 x 5632, batch 1, fp16 activations).
A step is one decode token's MLP matvecs over `--copies` distinct weight sets
(default 32, 623 MB), so every step streams its weights from HBM rather than
from the 256 MB Infinity Cache.  Per weight set, gate and up read the same
activations and run as one grouped launch, down as a second; the 2 x copies
launches are captured once in a HIP graph and replayed.  Inputs are resident in HBM before timing starts.

Algorithmic bytes of one matvec = packed weights including scales / zeros
(4.5 bits per weight) + activations read + outputs written; the dense
matrix the method never forms is not counted.  Per the pages' roofline
method (zynfer PR 100, stage M1/M2 profile notes: bytes per token against
streamed bandwidth), GB/s = bytes / time.

Also reported (`extras`): single-launch and cold-stream rates of the other
workloads (Q8_0 512x512, Q4K 0.6B MLP and 151936-row vocab head, the full
155-matvec 1.1B decode sweep at batch 1 and 8 -- grouped, with the fused
epilogues, and with 8-bit activation blocks -- the W4A16 prefill GEMM at
M = 16 / 128 / 512 in TFLOP/s), each with its fraction of peak and
tokens-equivalent rate (`gated` collects the roofline-gated ones), platform
probes, and the CPU oracle timed on the host (`cpu_baseline`: per config,
median of 3, dequantization and product split, and one BLAS thread).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--copies C]
                       [--no-extras] [--no-cpu-baseline] [--cpu-quick] [--leg NAME]
(--leg runs extras workloads alone and prints their results, for profiling.)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
# Tokens-equivalent per second (bytes-per-token roofline method, zynfer PR 100,
# stage M2): a matvec figure in GB/s divided by the bytes of one decode token of
# the 1.1B decoder (packed weights of its 155 matvecs); a GEMM figure in
# TFLOP/s divided by 2 flops per weight of that model.
TOKEN_BYTES_1B1 = 667_152_384
TOKEN_FLOPS_1B1 = 2 * 1_034_420_224
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
FP32_VALU_PEAK_TFLOPS = 157.3  # MI355X fp32 vector, published

# The source pages' own figures, each with the hardware it was measured on:
# context for the report, not targets and not comparable one to one (other
# machines, whole-model runs with attention and sampling included).
PAGES_CONTEXT = [
    {"figure": "CPU decode, TinyLlama-1.1B / Llama-3.2-1B, Q4_K_M weights, 8-bit activations, batch 1",
     "value": "128 / 113 tok/s", "hardware": "Apple M1 Pro, 8 threads (NEON dot product)",
     "source": "aot-llm README, benchmark figures"},
    {"figure": "Metal decode, same models, f32 activations, weights dequantized on the fly",
     "value": "106 / 92 tok/s", "hardware": "Apple M1 Pro GPU", "source": "aot-llm README, Metal backend notes"},
    {"figure": "Metal quantized matvec bandwidth, 1B-class decode", "value": "75-107 GB/s",
     "hardware": "Apple M1 Pro GPU", "source": "aot-llm README, Metal backend notes"},
    {"figure": "Metal prompt evaluation (batched, the prefill analogue), ~300-token prompts",
     "value": "550-750 tok/s", "hardware": "Apple M1 Pro GPU", "source": "aot-llm README, benchmark figures"},
    {"figure": "Qwen3-0.6B decode time per token: f32 / bf16 / per-row int8 weights",
     "value": "231-234 / 252-254 / 119 ms", "hardware": "Apple M-series laptop, Metal (STREAM ~228 GB/s)",
     "source": "zynfer PR 100, stages M2, M4 and M5"},
]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--copies", type=int, default=32)
    p.add_argument("--no-extras", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-quick", action="store_true",
                   help="skip the oracle's decode-token run (c5) in the CPU baseline")
    p.add_argument("--leg", default=None,
                   help="run only these extras workloads (comma-separated) and print their results "
                        "(profiling); of: "
                        + ", ".join(LEGS))
    return p.parse_args()


# ----------------------------------------------------------------- helpers

def _dev(a):
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def _x_dev(x, dtype):
    import torch
    t = _dev(x)
    return t if dtype == "f32" else t.view(torch.float16 if dtype == "f16" else torch.bfloat16)


def matvec_bytes(fmt, N, K, batch, x_bytes_per_el):
    import workloads as wl
    return int(round(wl.bytes_per_weight(fmt) * N * K)) + batch * K * x_bytes_per_el + batch * N * 4


REPLAY_STATS = {}  # per-replay statistics of the last time_graph call (median / min / p90 ms)


def time_graph(fn, steps, warmup, stream=None):
    """Capture fn() once into a HIP graph, replay warmup + steps times; ms per
    replay over the timed replays (one event before and one after them).  Then
    `steps` more replays with an event after each give the median, min and p90
    of single replays (REPLAY_STATS; the markers are kept out of the timed pass)."""
    import torch
    s = stream or torch.cuda.Stream()
    fn()  # eager once (argument checks, lazy init)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(s)
        for _ in range(steps):
            g.replay()
        t1.record(s)
    t1.synchronize()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    with torch.cuda.stream(s):
        ev[0].record(s)
        for i in range(steps):
            g.replay()
            ev[i + 1].record(s)
    ev[-1].synchronize()
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    REPLAY_STATS.clear()
    REPLAY_STATS.update({"replays": steps, "median_ms": per[len(per) // 2], "min_ms": per[0],
                         "p90_ms": per[min(len(per) - 1, (9 * len(per)) // 10)]})
    return ms, g


class Stream:
    """A set of distinct packed copies of some matrices, with per-copy x / y buffers."""

    def __init__(self, qmv, mats, x_dtype, batch, copies):
        import workloads as wl
        self.qmv, self.mats, self.x_dtype, self.batch = qmv, mats, x_dtype, batch
        self.logical = {}
        self.items = []  # (fmt, N, K, W, x, y)
        packed = {}
        for name, fmt, N, K, key in mats:
            w = wl.gen_weights(fmt, N, K, key)
            self.logical[name] = (fmt, w, wl.gen_x(K, batch, x_dtype, key))
            packed[name] = qmv.pack(fmt, {k: _dev(v) for k, v in w.items()})
        for c in range(copies):
            for name, fmt, N, K, key in mats:
                W = packed[name] if c == 0 else packed[name].clone()
                x = _x_dev(wl.gen_x(K, batch, x_dtype, (key[0], key[1], key[2], 77, c)), x_dtype)
                y = self._out(N)
                self.items.append((fmt, N, K, W, x, y))
        xb = {"f32": 4, "f16": 2, "bf16": 2}[x_dtype]
        self.bytes = sum(matvec_bytes(f, N, K, batch, xb) for f, N, K, *_ in self.items)
        self.launches = len(self.items)

    def _out(self, N):
        import torch
        return torch.empty((self.batch, N), dtype=torch.float32, device="cuda")

    def __call__(self):
        mv = self.qmv.matvec
        for fmt, N, K, W, x, y in self.items:
            mv(fmt, W, x, N, K, y=y)


# ------------------------------------------------------------------ legs

class MlpStream:
    """One decode token's MLP matvecs over `copies` distinct weight sets (each a
    layer's gate / up / down, packed once and cloned): per layer, gate and up
    read the same activations and run as one grouped launch, down as another."""

    def __init__(self, qmv, cfg, copies):
        import torch
        import workloads as wl
        self.qmv, self.x_dtype, self.mats = qmv, cfg["x_dtype"], cfg["mats"]
        (_, fmt, F, D, kg), (_, _, _, _, ku), (_, _, _, _, kd) = cfg["mats"]
        self.fmt, self.F, self.D = fmt, F, D
        self.logical = {}
        packed = {}
        for name, f, N, K, key in cfg["mats"]:
            w = wl.gen_weights(f, N, K, key)
            self.logical[name] = (f, w, wl.gen_x(K, 1, self.x_dtype, key))
            packed[name] = qmv.pack(f, {k: _dev(v) for k, v in w.items()})
        self.layers = []
        for c in range(copies):
            W = {n: packed[n] if c == 0 else packed[n].clone() for n in packed}
            xi = _x_dev(wl.gen_x(D, 1, self.x_dtype, (kg[0], kg[1], kg[2], 77, c)), self.x_dtype)
            xm = _x_dev(wl.gen_x(F, 1, self.x_dtype, (kd[0], kd[1], kd[2], 77, c)), self.x_dtype)
            ys = [torch.empty((1, n), dtype=torch.float32, device="cuda") for n in (F, F, D)]
            self.layers.append((W["gate"], W["up"], W["down"], xi, xm, ys))
        xb = 2 if self.x_dtype == "f16" else 4
        self.gate_up_bytes = gate_up_bytes(fmt, F, D, xb)
        self.down_bytes = matvec_bytes(fmt, D, F, 1, xb)
        self.bytes = copies * (self.gate_up_bytes + self.down_bytes)
        self.launches = 2 * copies

    def gate_up(self, layer):
        Wg, Wu, _, xi, _, (yg, yu, _) = layer
        self.qmv.matvec_grouped(self.fmt, [(Wg, xi, self.F, yg), (Wu, xi, self.F, yu)], self.D)

    def down(self, layer):
        _, _, Wd, _, xm, (_, _, yd) = layer
        self.qmv.matvec(self.fmt, Wd, xm, self.D, self.F, y=yd)

    def __call__(self):
        for layer in self.layers:
            self.gate_up(layer)
            self.down(layer)

    def ungrouped(self):
        """The same work as three single matvecs per layer (for comparison)."""
        mv = self.qmv.matvec
        for Wg, Wu, Wd, xi, xm, (yg, yu, yd) in self.layers:
            mv(self.fmt, Wg, xi, self.F, self.D, y=yg)
            mv(self.fmt, Wu, xi, self.F, self.D, y=yu)
            mv(self.fmt, Wd, xm, self.D, self.F, y=yd)


def gate_up_bytes(fmt, F, D, xb):
    """Algorithmic bytes of the grouped gate + up launch: both matrices, the
    shared activations once, both outputs."""
    import workloads as wl
    return 2 * int(round(wl.bytes_per_weight(fmt) * F * D)) + D * xb + 2 * F * 4


def headline(qmv, args):
    import workloads as wl
    st = MlpStream(qmv, wl.c2_w4a16_mlp(), args.copies)
    ms, _ = time_graph(st, args.steps, args.warmup)
    st.replay_stats = dict(REPLAY_STATS)
    gbs = st.bytes / (ms * 1e-3) / 1e9
    return st, ms, gbs


def kernel_leg(qmv, st, steps, warmup):
    """Per-launch duration of each launch of the headline step: a graph of the
    launches of one kind over all cold copies, back to back, timed with events
    on the stream they run on."""
    out = {}
    for tag, fn, b in (("gate+up grouped", st.gate_up, st.gate_up_bytes), ("down", st.down, st.down_bytes)):
        def run(fn=fn):
            for layer in st.layers:
                fn(layer)
        ms, _ = time_graph(run, steps, warmup)
        per = ms / len(st.layers)
        out[tag] = {"us_per_launch": per * 1e3, "bytes_per_launch": b,
                    "gbs": b / (per * 1e-3) / 1e9, "launches": len(st.layers)}
    ms, _ = time_graph(st.ungrouped, steps, warmup)
    out["step_ungrouped"] = {"ms_per_step": ms, "gbs": st.bytes / (ms * 1e-3) / 1e9,
                             "launches": 3 * len(st.layers)}
    return out


# Source files of the matvec kernels the headline launches, and the kernel
# instantiation the dispatcher picks for the grouped gate / up launch (fp16 x,
# K = 2048: 64 lanes per row, one unit per lane, four rows per lane group, two
# segments in a 4-entry table, K not split, one row group per wave).
MATVEC_SOURCES = ["gemm_dequant_matvec_amd/csrc/matvec_xs.hip", "gemm_dequant_matvec_amd/csrc/qmv_internal.h"]
GATE_KERNEL = "matvec_xs_kernel<2, true, 64, 1, 4, 4, 1, false>"


def measured_traffic(profile: str, kernel: str):
    """HBM bytes per dispatch from the committed counter summary, or None when the
    kernel sources changed since the counters were taken (or none were taken)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))[profile]
        h = hashlib.sha256()
        for f in rec["sources"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if h.hexdigest()[:16] != rec["source_sha"]:
            return None
        return rec["kernels"][kernel]["bytes"]
    except (OSError, KeyError, ValueError):
        return None


def copy_probe():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(10):
        b.copy_(a)
    t1.record()
    t1.synchronize()
    ms = t0.elapsed_time(t1) / 10
    del a, b
    return {"bytes": 2 * n, "gbs": 2 * n / (ms * 1e-3) / 1e9, "what": "torch copy_ of 1 GiB (read+write)"}


def platform_probes(qmv):
    """The machine's own ceilings, for reading the other figures: device-copy GB/s
    (read + write) at 16 MiB .. 4 GiB (past the 256 MB Infinity Cache from 256 MiB
    up), and the cost of one tiny kernel launch, eager and inside a HIP graph."""
    import torch
    out = {"copy_gbs": {}}
    for mib in (16, 64, 256, 1024, 4096):
        n = mib << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        reps = 20 if mib <= 256 else 5
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            b.copy_(a)
        t1.record()
        t1.synchronize()
        ms = t0.elapsed_time(t1) / reps
        out["copy_gbs"][f"{mib}MiB"] = 2 * n / (ms * 1e-3) / 1e9
        del a, b
    z = torch.zeros(1, device="cuda")
    n_launch = 200

    def tiny():
        for _ in range(n_launch):
            z.fill_(1.0)
    tiny()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    tiny()
    t1.record()
    t1.synchronize()
    out["launch_us_eager"] = t0.elapsed_time(t1) * 1e3 / n_launch
    ms, _ = time_graph(tiny, 10, 3)
    out["launch_us_graph"] = ms * 1e3 / n_launch
    out["what"] = "torch copy_ per size; launch: one-element fill kernel, 200 back to back"
    return out


def _gbs_result(d, gbs):
    d.update({"gbs": gbs, "frac_hbm": gbs / HBM_PEAK_GBS, "replays": dict(REPLAY_STATS),
              "tok_per_s_equiv": gbs * 1e9 / TOKEN_BYTES_1B1,
              "tok_note": "GB/s / bytes of one 1.1B decode token (667152384 B)"})
    return d


def leg_q8_0(qmv):
    """Q8_0 512x512: one launch, latency-bound (same matrix 20x back to back)."""
    import workloads as wl
    st = Stream(qmv, wl.c1_q8_0()["mats"], "f32", 1, 1)
    ms, _ = time_graph(lambda: [st() for _ in range(20)], 20, 5)
    ms /= 20
    return _gbs_result({"us": ms * 1e3, "note": "same matrix 20x back to back (cache-warm, latency-bound)"},
                       st.bytes / (ms * 1e-3) / 1e9)


def leg_mlp06(qmv):
    """Q4K 0.6B MLP up / down, 170 cold copies of each (608 MB)."""
    import workloads as wl
    mlp = [m for m in wl.c3_q4k_0b6()["mats"] if m[0] != "head"]
    st = Stream(qmv, mlp, "f32", 1, 170)
    ms, _ = time_graph(st, 20, 3)
    return _gbs_result({"us_per_launch": ms * 1e3 / st.launches, "launches": st.launches},
                       st.bytes / (ms * 1e-3) / 1e9)


def leg_head06(qmv):
    """The 151936 x 1024 Q4K vocab head, 8 cold copies (705 MB)."""
    import workloads as wl
    head = [m for m in wl.c3_q4k_0b6()["mats"] if m[0] == "head"]
    st = Stream(qmv, head, "f32", 1, 8)
    ms, _ = time_graph(st, 20, 3)
    return _gbs_result({"us_per_launch": ms * 1e3 / st.launches, "bytes_per_launch": st.bytes // st.launches},
                       st.bytes / (ms * 1e-3) / 1e9)


def leg_stream_ramp(qmv):
    """Launch time against launch size: the grouped W4A16 gate+up launch (two
    matrices of 5632 c x 2048, fp16 x, batch 1) at c = 1, 2, 4, 8, over enough
    cold copies to stream >= 700 MB per graph.  The line t = t0 + bytes / bw
    fitted to the per-launch times splits a launch into a fixed part (launch,
    first-load latency, drain) and the steady streaming rate."""
    import numpy as np
    import torch
    import workloads as wl
    K, pts = 2048, []
    for c in (1, 2, 4, 8):
        N = 5632 * c
        mats = []
        for i in range(2):
            w = wl.gen_weights("w4a16_g64", N, K, (9, c, i))
            mats.append(qmv.pack("w4a16_g64", {k: _dev(v) for k, v in w.items()}))
        nbytes = gate_up_bytes("w4a16_g64", N, K, 2)
        copies = max(2, -(-700_000_000 // nbytes))
        x = _x_dev(wl.gen_x(K, 1, "f16", (9, c, 9)), "f16")
        calls = []
        for j in range(copies):
            Ws = mats if j == 0 else [m.clone() for m in mats]
            ys = [torch.empty((1, N), dtype=torch.float32, device="cuda") for _ in range(2)]
            calls.append([(Ws[0], x, N, ys[0]), (Ws[1], x, N, ys[1])])

        def run(calls=calls):
            for items in calls:
                qmv.matvec_grouped("w4a16_g64", items, K)
        ms, _ = time_graph(run, 10, 3)
        us = ms * 1e3 / copies
        pts.append({"rows_per_matrix": N, "bytes": nbytes, "us": us, "gbs": nbytes / (us * 1e-6) / 1e9})
        del calls, mats
        torch.cuda.empty_cache()
    b = np.array([p["bytes"] for p in pts], dtype=np.float64)
    t = np.array([p["us"] for p in pts], dtype=np.float64)
    slope, t0 = np.polyfit(b, t, 1)
    return {"points": pts, "fit_t0_us": t0, "fit_steady_gbs": 1e-3 / slope,
            "note": "t = t0 + bytes / steady_gbs, least squares over the four sizes"}


def _sweep_result(ms, b, nbytes, launches, matvecs):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms_per_token_step": ms, "tok_per_s": b / (ms * 1e-3), "gbs": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
            "bytes": nbytes, "launches": launches, "matvecs": matvecs, "replays": dict(REPLAY_STATS)}


def leg_sweep(qmv, b):
    """One decode token of the 1.1B decoder at batch b: 155 matvecs, 667 MB of weights."""
    import workloads as wl
    st = Sweep(qmv, wl.c5_sweep(b), b)
    ms, _ = time_graph(st, 20, 3)
    return _sweep_result(ms, b, st.bytes, st.launches, st.matvecs)


def leg_sweep_q8x(qmv, b):
    """The same token with the integer-dot variant: each distinct activation
    vector quantized once per step (included in the time), integer dot products."""
    import workloads as wl
    st = Sweep(qmv, wl.c5_sweep(b), b)
    step = st.with_q8x()
    ms, _ = time_graph(step, 20, 3)
    r = _sweep_result(ms, b, step.bytes, step.launches, st.matvecs)
    r["note"] = "bytes as the f32 sweep; launches include one quantize per distinct x"
    return r


def leg_sweep_fused(qmv, b):
    """The token with fused epilogues: o and down add the residual in place,
    gate / up / SwiGLU in one pass (h written once)."""
    import workloads as wl
    st = FusedSweep(qmv, wl.c5_sweep(b), b)
    ms, _ = time_graph(st, 20, 3)
    return _sweep_result(ms, b, st.bytes, st.launches, st.matvecs)


LEGS = {
    "platform_probes": platform_probes,
    "copy_probe_1GiB": lambda q: copy_probe(),
    "q8_0_512x512_b1_single": leg_q8_0,
    "q4k_0.6B_mlp_b1_cold": leg_mlp06,
    "q4k_vocab_head_151936x1024_b1_cold": leg_head06,
    "stream_ramp_w4a16_gate_up_b1": leg_stream_ramp,
    "decode_sweep_1.1B_b1": lambda q: leg_sweep(q, 1),
    "decode_sweep_1.1B_b8": lambda q: leg_sweep(q, 8),
    "decode_sweep_1.1B_b1_fused": lambda q: leg_sweep_fused(q, 1),
    "decode_sweep_1.1B_b8_fused": lambda q: leg_sweep_fused(q, 8),
    "decode_sweep_1.1B_b1_q8x": lambda q: leg_sweep_q8x(q, 1),
    "decode_sweep_1.1B_b8_q8x": lambda q: leg_sweep_q8x(q, 8),
    "gemm_w4a16_M16": lambda q: gemm_leg(q, 16),
    "gemm_w4a16_M128": lambda q: gemm_leg(q, 128),
    "gemm_w4a16_M512": lambda q: gemm_leg(q, 512),
}


def extras(qmv, args):
    res = {}
    for name, fn in LEGS.items():
        try:
            res[name] = fn(qmv)
        except Exception as e:  # a leg that cannot run is reported, not faked
            res[name] = {"error": str(e)[:200]}
    return res


class Sweep:
    """The 155 matvecs of one decode token: distinct shapes generated once, every
    layer gets its own device copy (so the 667 MB sweep streams from HBM).
    Matrices that read the same activations and share a format (or are all
    Q4K / Q6K) run as one grouped call: q + k (Q4K) + v (Q6K), gate + up; o,
    down and the head alone."""

    SHARED = {"q": "attn_in", "k": "attn_in", "v": "attn_in", "gate": "mlp_in", "up": "mlp_in"}

    def __init__(self, qmv, cfg, batch):
        import torch
        import workloads as wl
        self.qmv, self.batch = qmv, batch
        shapes, xs = {}, {}
        self.calls = []  # (fmt or None when mixed, K, [(W, x, N, y, fmt), ...])
        prev = None
        self.bytes = 0
        for name, fmt, N, K, key in cfg["mats"]:
            tag = (fmt, N, K)
            if tag not in shapes:
                w = wl.gen_weights(fmt, N, K, key)
                shapes[tag] = W = qmv.pack(fmt, {k: _dev(v) for k, v in w.items()})
            else:
                W = shapes[tag].clone()
            layer, nm = name.split(".") if "." in name else ("", name)
            share = (layer, self.SHARED.get(nm, nm))
            if share not in xs:
                xs[share] = _x_dev(wl.gen_x(K, batch, "f32", key), "f32")
                self.bytes += batch * K * 4
            y = torch.empty((batch, N), dtype=torch.float32, device="cuda")
            self.bytes += int(round(wl.bytes_per_weight(fmt) * N * K)) + batch * N * 4
            item = (W, xs[share], N, y, fmt)
            fmts = {fmt} | ({it[4] for it in self.calls[-1][2]} if prev == (share, K) else set())
            if prev == (share, K) and (len(fmts) == 1 or fmts <= {"q4k", "q6k"}):
                _, _, items = self.calls[-1]
                self.calls[-1] = (fmt if len(fmts) == 1 else None, K, items + [item])
            else:
                self.calls.append((fmt, K, [item]))
            prev = (share, K)
        self.launches = len(self.calls)
        self.matvecs = sum(len(c[2]) for c in self.calls)

    def __call__(self):
        for fmt, K, items in self.calls:
            if len(items) == 1:
                W, x, N, y, _ = items[0]
                self.qmv.matvec(fmt, W, x, N, K, y=y)
            else:
                self.qmv.matvec_grouped(fmt, items, K)

    def with_q8x(self):
        """The integer-dot variant of the same sweep: every distinct activation
        vector is quantized to 8-bit blocks once (qmv_quantize_x, inside the
        step), and each matvec reads the quantized copy."""
        bufs, calls = {}, []
        for fmt, K, items in self.calls:
            new = []
            for W, x, N, y, f in items:
                if id(x) not in bufs:
                    bufs[id(x)] = (x, self.qmv.quantize_x(x))
                new.append((W, bufs[id(x)][1], N, y, f))
            calls.append((fmt, K, new))
        pairs = list(bufs.values())
        qmv = self.qmv
        # quantize each distinct vector right before its first use
        first_use = {}
        for ci, (fmt, K, items) in enumerate(calls):
            for W, xq, N, y, f in items:
                first_use.setdefault(id(xq), ci)
        quant_at = {}
        for x, xq in pairs:
            quant_at.setdefault(first_use[id(xq)], []).append((x, xq))

        def step():
            for ci, (fmt, K, items) in enumerate(calls):
                for x, xq in quant_at.get(ci, ()):
                    qmv.quantize_x(x, out=xq.data)
                if len(items) == 1:
                    W, xq, N, y, _ = items[0]
                    qmv.matvec(fmt, W, xq, N, K, y=y)
                else:
                    qmv.matvec_grouped(fmt, items, K)
        step.launches = len(calls) + len(pairs)
        step.bytes = self.bytes  # the same algorithmic bytes as the f32 sweep
        return step


class FusedSweep:
    """One decode token of the 1.1B decoder with the fused epilogues: per layer
    q + k + v grouped; o with the residual add fused (the residual stream is
    updated in place); gate / up / SwiGLU in one pass writing h; down reading h
    with the residual add fused; then the vocab head.  Four launches per layer
    plus the head, as in the grouped sweep, but the MLP writes one vector
    instead of two and no separate add runs.  Every layer has its own device
    copy of the weights (distinct shapes generated once, then cloned)."""

    def __init__(self, qmv, cfg, batch):
        import torch
        import workloads as wl
        self.qmv, self.batch = qmv, batch
        packed, shapes = {}, {}
        for name, fmt, N, K, key in cfg["mats"]:
            tag = (fmt, N, K)
            if tag not in shapes:
                w = wl.gen_weights(fmt, N, K, key)
                shapes[tag] = qmv.pack(fmt, {k: _dev(v) for k, v in w.items()})
                packed[name] = shapes[tag]
            else:
                packed[name] = shapes[tag].clone()
        f32 = dict(dtype=torch.float32, device="cuda")
        D, F = wl.LLAMA_1B1["dim"], wl.LLAMA_1B1["mlp"]
        gx = lambda K, k: _x_dev(wl.gen_x(K, batch, "f32", (5, 2000, k)), "f32")
        self.resid = gx(D, 0)
        self.layers = []
        nbytes = 0
        n_layers = sum(1 for m in cfg["mats"] if m[0].endswith(".q"))
        for L in range(n_layers):
            W = {nm: packed[f"l{L}.{nm}"] for nm in ("q", "k", "v", "o", "gate", "up", "down")}
            lay = dict(W=W, attn_in=gx(D, 10 * L + 1), o_in=gx(D, 10 * L + 2), mlp_in=gx(D, 10 * L + 3),
                       q=torch.empty((batch, D), **f32), k=torch.empty((batch, 256), **f32),
                       v=torch.empty((batch, 256), **f32), h=torch.empty((batch, F), **f32))
            self.layers.append(lay)
        for name, fmt, N, K, key in cfg["mats"]:
            nbytes += int(round(wl.bytes_per_weight(fmt) * N * K))
        V = wl.LLAMA_1B1["vocab"]
        self.head = (packed["head"], gx(D, 9999), torch.empty((batch, V), **f32), V)
        xb, L = batch * 4, n_layers
        # activations: per layer attn_in, o_in, mlp_in, h read; q, k, v, h written;
        # residual read + written twice; head x in, logits out
        nbytes += L * xb * (3 * D + F + (D + 256 + 256 + F) + 4 * D) + xb * (D + V)
        self.bytes = nbytes
        self.launches = 4 * L + 1
        self.matvecs = 7 * L + 1

    def __call__(self):
        qmv, r = self.qmv, self.resid
        D, F = r.shape[1], self.layers[0]["h"].shape[1]
        for lay in self.layers:
            W = lay["W"]
            qmv.matvec_grouped(None, [(W["q"], lay["attn_in"], D, lay["q"], "q4k"),
                                      (W["k"], lay["attn_in"], 256, lay["k"], "q4k"),
                                      (W["v"], lay["attn_in"], 256, lay["v"], "q6k")], D)
            qmv.matvec_ex("q4k", W["o"], lay["o_in"], D, D, y=r, residual=r)
            qmv.matvec_swiglu("q4k", W["gate"], W["up"], lay["mlp_in"], F, D, h=lay["h"])
            qmv.matvec_ex("q6k", W["down"], lay["h"], D, F, y=r, residual=r)
        Wh, xh, yh, V = self.head
        qmv.matvec("q6k", Wh, xh, V, D, y=yh)


def gemm_leg(qmv, M, reps=20):
    """Prefill GEMM time per launch: a graph of `reps` back-to-back launches, so the
    graph-launch overhead of one replay is spread over many kernels."""
    import torch
    import workloads as wl
    c4 = wl.c4_gemm(M)
    name, fmt, N, K, key = c4["mats"][0]
    w = wl.gen_weights(fmt, N, K, key)
    W = qmv.pack(fmt, {k: _dev(v) for k, v in w.items()})
    X = _x_dev(wl.gen_x(K, M, "bf16", key), "bf16")
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def run():
        for _ in range(reps):
            qmv.gemm(fmt, W, X, N, K, Y=Y)
    ms, _ = time_graph(run, 20, 3)
    rs = dict(REPLAY_STATS)  # per replay of `reps` launches
    ms /= reps
    flops = 2.0 * M * N * K
    tf = flops / (ms * 1e-3) / 1e12
    # the matvec path run at batch = M, for the crossover
    Xf = X.float()
    ymv = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def run_mv():
        for _ in range(reps):
            qmv.matvec(fmt, W, Xf, N, K, y=ymv)
    ms_mv, _ = time_graph(run_mv, 5, 2)
    ms_mv /= reps
    # context: the vendor bf16 GEMM (torch.matmul -> hipBLASLt) on the same matrix
    # dequantized to a dense bf16 copy (3.5x the weight bytes; not this library's path)
    # (a contiguous [K][N] copy: no transposed view is handed to the library)
    WdT = qmv.dequant(fmt, W, N, K).to(torch.bfloat16).t().contiguous()
    Yd = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def run_blas():
        for _ in range(reps):
            torch.matmul(X, WdT, out=Yd)
    ms_bl, _ = time_graph(run_blas, 5, 2)
    ms_bl /= reps
    del WdT
    return {"us": ms * 1e3, "tflops": tf, "frac_bf16_peak": tf / BF16_PEAK_TFLOPS,
            "tok_per_s": M / (ms * 1e-3), "prefill_tok_per_s_equiv": tf * 1e12 / TOKEN_FLOPS_1B1,
            "replays_of_20_launches": rs,
            "matvec_path_us": ms_mv * 1e3, "dense_bf16_library_gemm_us": ms_bl * 1e3,
            "dense_bf16_library_frac_peak": flops / (ms_bl * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_matvecs(oracle, mats, reps=1):
    """Dequantize + f64 product of each (fmt, w, x) `reps` times; (dequant s, product s)."""
    import numpy as np
    t_dq = t_mv = 0.0
    for _ in range(reps):
        for fmt, w, x, xdt in mats:
            t0 = time.perf_counter()
            W = oracle.dequant(fmt, w)
            t1 = time.perf_counter()
            xv = oracle.f16_to_f64(x) if xdt == "f16" else x.astype(np.float64)
            oracle.matvec_ref(W, xv)
            t_mv += time.perf_counter() - t1
            t_dq += t1 - t0
            del W
    return t_dq, t_mv


def cpu_baseline(args):
    """The oracle, untuned, on the host: numpy f32 dequantization (one thread)
    and the f64 product (BLAS, as many threads as cores this process may use).
    Per config the median of 3 runs (the decode token: 3 when one takes under
    5 s, else 1), split into
    dequantization and product time; c1-c3 also with one BLAS thread.  Inputs
    are generated before timing.  `value` is the headline workload's rate."""
    import statistics
    import numpy as np
    import oracle
    import workloads as wl
    from threadpoolctl import threadpool_limits
    cores = len(os.sched_getaffinity(0))

    def mats_of(cfg):
        xdt = cfg["x_dtype"]
        return [(fmt, wl.gen_weights(fmt, N, K, key), wl.gen_x(K, cfg["batch"], xdt, key), xdt)
                for _, fmt, N, K, key in cfg["mats"]]

    def cfg_bytes(cfg):
        xb = {"f32": 4, "f16": 2, "bf16": 2}[cfg["x_dtype"]]
        return sum(matvec_bytes(fmt, N, K, cfg["batch"], xb) for _, fmt, N, K, _ in cfg["mats"])

    def timed(mats, nbytes, runs):
        res = [_oracle_matvecs(oracle, mats) for _ in range(runs)]
        tot = [a + b for a, b in res]
        med = statistics.median(tot)
        k = tot.index(med) if med in tot else 0
        return {"s": med, "dequant_s": res[k][0], "product_s": res[k][1], "runs": runs,
                "gbs": nbytes / med / 1e9}

    per = {}
    t_start = time.perf_counter()
    cfgs = {"c1_q8_0_512x512_b1": wl.c1_q8_0(), "c2_w4a16_1.1B_mlp_b1": wl.c2_w4a16_mlp(),
            "c3_q4k_0.6B_mlp_head_b1": wl.c3_q4k_0b6()}
    with threadpool_limits(limits=cores):
        for tag, cfg in cfgs.items():
            per[tag] = timed(mats_of(cfg), cfg_bytes(cfg), 3)
        # c4: the GEMM at M = 512 (dequantize + f64 X W^T)
        _, fmt, N, K, key = wl.c4_gemm(512)["mats"][0]
        w, X = wl.gen_weights(fmt, N, K, key), oracle.bf16_to_f64(wl.gen_x(K, 512, "bf16", key))
        runs = []
        for _ in range(3):
            t0 = time.perf_counter()
            W = oracle.dequant(fmt, w)
            t1 = time.perf_counter()
            oracle.gemm_ref(W, X)
            runs.append((t1 - t0, time.perf_counter() - t1))
        tot = sorted(runs, key=lambda r: r[0] + r[1])[1]
        per["c4_w4a16_gemm_M512"] = {"s": tot[0] + tot[1], "dequant_s": tot[0], "product_s": tot[1], "runs": 3,
                                     "tflops": 2.0 * 512 * N * K / (tot[0] + tot[1]) / 1e12}
        if not args.cpu_quick:
            # c5: one decode token at batch 1 (distinct shapes generated once, each run as many
            # times as the token has such matrices; the oracle's time does not depend on values)
            cfg = wl.c5_sweep(1)
            counts, first = {}, {}
            for name, fmt, N, K, key in cfg["mats"]:
                counts[(fmt, N, K)] = counts.get((fmt, N, K), 0) + 1
                first.setdefault((fmt, N, K), key)
            shapes = [(fmt, wl.gen_weights(fmt, N, K, key), wl.gen_x(K, 1, "f32", key), "f32")
                      for (fmt, N, K), key in first.items()]

            def token():
                t_dq = t_mv = 0.0
                for m in shapes:
                    N, K = m[1]["q"].shape
                    a, b = _oracle_matvecs(oracle, [m], reps=counts[(m[0], N, K)])
                    t_dq, t_mv = t_dq + a, t_mv + b
                return t_dq, t_mv
            runs = [token()]
            if sum(runs[0]) < 5.0:  # a fast host: the median of 3 still fits the time budget
                runs += [token(), token()]
            t_dq, t_mv = sorted(runs, key=sum)[len(runs) // 2]
            per["c5_decode_token_1.1B_b1"] = {"s": t_dq + t_mv, "dequant_s": t_dq, "product_s": t_mv,
                                              "runs": len(runs), "tok_per_s": 1.0 / (t_dq + t_mv),
                                              "gbs": cfg_bytes(cfg) / (t_dq + t_mv) / 1e9}
    one = {}
    with threadpool_limits(limits=1):
        for tag, cfg in cfgs.items():
            one[tag] = timed(mats_of(cfg), cfg_bytes(cfg), 1)
    head = per["c2_w4a16_1.1B_mlp_b1"]
    return {"value": head["gbs"], "unit": "GB/s", "cores": cores, "kind": "oracle",
            "cpu_model": _cpu_model(), "blas_threads": cores,
            "sample": "headline workload (one 1.1B MLP layer: gate, up, down, W4A16 g64, b=1, fp16 x), "
                      "median of 3: numpy f32 dequant (1 thread) + f64 matvec (BLAS); "
                      f"whole baseline {time.perf_counter() - t_start:.1f} s",
            "per_config": per, "one_blas_thread": one,
            "note": "correctness oracle, not a tuned CPU kernel"}


def gated_figures(out):
    """The figures held against the roofline: the 1.1B decode token at batch 1
    (grouped and fused), the 151936-row vocab head and the W4A16 MLP stream
    against HBM; the W4A16 GEMM at M = 512 against bf16 MFMA; each with its
    tokens-equivalent rate."""
    ex = out.get("extras", {})
    g = {"c2_w4a16_mlp_stream_b1": {"gbs": out["value"], "frac_hbm": out["value"] / HBM_PEAK_GBS,
                                    "tok_per_s_equiv": out["value"] * 1e9 / TOKEN_BYTES_1B1}}
    for tag, leg in (("c5_decode_token_b1", "decode_sweep_1.1B_b1"),
                     ("c5_decode_token_b1_fused", "decode_sweep_1.1B_b1_fused"),
                     ("c5_decode_token_b8", "decode_sweep_1.1B_b8"),
                     ("c3_q4k_vocab_head", "q4k_vocab_head_151936x1024_b1_cold")):
        r = ex.get(leg, {})
        if "gbs" in r:
            g[tag] = {"gbs": r["gbs"], "frac_hbm": r["gbs"] / HBM_PEAK_GBS,
                      "tok_per_s" if "tok_per_s" in r else "tok_per_s_equiv":
                          r.get("tok_per_s", r.get("tok_per_s_equiv"))}
    r = ex.get("stream_ramp_w4a16_gate_up_b1", {})
    if "fit_steady_gbs" in r:
        g["gate_up_launch_steady_state"] = {"fixed_us_per_launch": r["fit_t0_us"], "gbs": r["fit_steady_gbs"],
                                            "frac_hbm": r["fit_steady_gbs"] / HBM_PEAK_GBS}
    r = ex.get("gemm_w4a16_M512", {})
    if "tflops" in r:
        g["c4_w4a16_gemm_M512"] = {"tflops": r["tflops"], "frac_bf16_mfma": r["frac_bf16_peak"],
                                   "tok_per_s": r["tok_per_s"],
                                   "prefill_tok_per_s_equiv": r["prefill_tok_per_s_equiv"]}
    return g


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(requested --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch
    import gemm_dequant_matvec_amd as qmv
    assert torch.cuda.is_available(), "no GPU visible"
    torch.cuda.set_device(0)
    if args.leg is not None:
        for leg in args.leg.split(","):
            if leg not in LEGS:
                print(f"unknown leg {leg!r}; one of {', '.join(LEGS)}", file=sys.stderr)
                sys.exit(2)
        for leg in args.leg.split(","):
            print(json.dumps({"leg": leg, "result": LEGS[leg](qmv)}), flush=True)
        return

    log("headline: W4A16 g64 1.1B MLP matvecs, batch 1, copies", args.copies)
    st, ms, gbs = headline(qmv, args)
    log(f"  {ms * 1e3:.1f} us/step, {gbs:.1f} GB/s")
    kl = kernel_leg(qmv, st, 20, 5)
    log("  per-shape:", json.dumps(kl))
    # the grouped gate / up launch: two thirds of the step's bytes and time
    dom_tag = "gate+up grouped"
    dom = kl[dom_tag]
    traffic = measured_traffic("matvec_w4a16_g64_1.1B_mlp_b1", GATE_KERNEL)
    roofline = {"bound": "hbm", "achieved": dom["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": dom["gbs"] / HBM_PEAK_GBS, "traffic": traffic,
                "kernel": f"{GATE_KERNEL} (gate+up grouped, 2 x 5632x2048)",
                "us_per_launch": dom["us_per_launch"], "bytes_per_launch": dom["bytes_per_launch"]}
    out = {
        "metric": "decode matvec achieved HBM GB/s (% of peak); prefill GEMM TFLOP/s",
        "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16*f16->f32", "data": "synthetic (seeded random blocks and activations, 1.1B-decoder shapes)",
        "config": {"workload": "W4A16-g64 decode matvec, 1.1B-decoder MLP (gate, up 5632x2048 "
                               "as one grouped launch; down 2048x5632), batch 1, fp16 x",
                   "copies": args.copies, "launches_per_step": st.launches,
                   "bytes_per_step": st.bytes, "frac_of_peak": gbs / HBM_PEAK_GBS,
                   "replays": st.replay_stats},
        "roofline": roofline,
    }
    log("copy probe")
    out["copy_probe"] = copy_probe()
    if not args.no_extras:
        log("extras")
        out["extras"] = extras(qmv, args)
        out["gated"] = gated_figures(out)
    out["pages_context"] = PAGES_CONTEXT
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
