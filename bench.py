#!/usr/bin/env python3
"""Bench of the small-T groupwise-int projection on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20]

A step is one projection Y = X . dequant(Wq) of the headline workload: the
GDN-QK-like int4 projection, T=8, K=5120, N=8192, group 64, fp16 scales, with
inputs resident in HBM.  Consecutive steps rotate through distinct weight
replicas totalling > 1 GiB, so every step streams its weights from HBM rather
than from the 256 MB Infinity Cache.  Steps are timed with HIP events on the
stream the kernels run on.  The line printed also carries the sweep the metric
asks for (T = 1, 2, 4, 8 for the int4 QK and int5 gate/value projections, and
the SwiGLU pair, the fused QK + gate/value + gate/up launch and the split-K
down projection), the stacked-layer sweep (64 layers of distinct weights,
eager and as replayed graphs), the roofline of the dominant kernel, and the
CPU leg: the oracle's own CPU time and, from the same oracle, the parity of
the timed configuration.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/projection + effective HBM GB/s (% of peak) at T=1,2,4,8, K=5120 int4/int5"
PEAK_GBS = 8000.0  # MI355X HBM3E peak
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA peak (prefill-size T is a dense contraction)
COLD_BYTES = 1 << 30
KERNEL_SRC = os.path.join(ROOT, "groupwise_int_weight_amd", "csrc", "ngq_gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="qk", choices=["qk", "gv"])
    p.add_argument("--T", type=int, default=8)
    p.add_argument("--no-sweep", action="store_true", help="time only the headline configuration")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-calibration", action="store_true")
    p.add_argument("--sweep-steps", type=int, default=100)
    p.add_argument("--no-stack", action="store_true", help="skip the stacked-layer sweep")
    p.add_argument("--stack-layers", type=int, default=64)
    p.add_argument("--stack-passes", type=int, default=5)
    p.add_argument("--stack-t", type=int, nargs="*", default=[1, 2, 4, 8], help="token counts of the stack sweep")
    p.add_argument("--no-stack-side", action="store_true", help="skip the side-stream comparison graph")
    p.add_argument("--fused", type=int, default=0, metavar="T",
                   help="time only the fused qk + gv + gate/up launch at T tokens (for profiling) and exit")
    p.add_argument("--valu-vs-mfma", action="store_true",
                   help="only the A/B of the streaming kernel's MFMA and VALU inner steps per bit width and T")
    p.add_argument("--ab-reps", type=int, default=5, help="interleaved repetitions of each A/B candidate")
    p.add_argument("--no-prefill", action="store_true", help="skip the prefill-size T sweep")
    p.add_argument("--prefill-t", type=int, nargs="*", default=[128, 256, 512, 1024, 2048],
                   help="token counts of the prefill sweep")
    p.add_argument("--no-cpu-configs", action="store_true",
                   help="skip the oracle's CPU time per workload and T (the headline's CPU baseline stays)")
    p.add_argument("--summarize-trace", metavar="CSV",
                   help="print per-kernel duration percentiles of a rocprofv3 kernel-trace CSV and exit (no GPU)")
    return p.parse_args()


def packed_bytes(ngq, w):
    return ngq.ngq_packed_bytes(w.K, w.N, w.bits)


def algorithmic_bytes(ngq, w, T, n_out=None):
    """Packed weights + scales read once, X read once, Y written once."""
    n_out = w.N if n_out is None else n_out
    return packed_bytes(ngq, w) + ngq.ngq_scale_bytes(w.K, w.N, w.bits) + 2 * T * w.K + 2 * T * n_out


class Rotation:
    """Distinct replicas of one workload's weights, enough to exceed the caches."""

    def __init__(self, ngq, w, T, seed=0):
        import synthetic

        self.w = w
        self.T = T
        nb = packed_bytes(ngq, w)
        per = nb + ngq.ngq_scale_bytes(w.K, w.N, w.bits)
        self.replicas = max(2, math.ceil(COLD_BYTES / per))
        self.wq, self.s, self.x = synthetic.device_replicas(w, T, self.replicas, nb, seed=seed)
        self.cold_bytes = self.replicas * per


# GPU clock cycles of the spin kernel queued ahead of the timed launches (at
# least ~2 ms: with ~0.4 ms, 20 QK launches timed 7.66 us each against 7.49,
# and varied more; 200 launches were unaffected), and the cycles per
# microsecond it is sized with
LEAD_CYCLES = 5_000_000
SPIN_CYCLES_PER_US = 2400


def time_steps(launch, replicas, steps, warmup):
    """Average GPU time of one launch: `warmup` eager launches (untimed; they
    also give the host's cost per launch), then exactly `steps` launches,
    rotating through the replicas, enqueued between two events on the
    launching stream behind a spin kernel that outlasts their submission (after
    one untimed pass of the same launches), so that the GPU runs them back to
    back with no host latency between them
    (checked: the host must have enqueued the last launch before the spin
    ended, else the spin is lengthened and the measurement taken again).
    Measured on MI355X (QK, T = 8): 20 such launches take 7.44 us each, the
    same 20 as one HIP graph replay 7.65 us (a replay adds ~9 us of its own:
    15.8 us for a graph of one launch); at 200 launches 7.43 eager and 7.22
    in a graph."""
    import torch

    t0 = time.perf_counter()
    for i in range(warmup):
        launch(i % replicas)
    host_us = (time.perf_counter() - t0) * 1e6 / max(1, warmup)
    # one untimed pass of the same launches settles the clocks (the first
    # timed pass of a process otherwise ran ~10 % slow)
    for i in range(steps):
        launch(i % replicas)
    torch.cuda.synchronize()
    spin = max(LEAD_CYCLES, int(4 * steps * host_us * SPIN_CYCLES_PER_US))
    for _ in range(3):
        e_spin = torch.cuda.Event(enable_timing=True)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        h0 = time.perf_counter()
        e_spin.record()
        torch.cuda._sleep(spin)
        start.record()
        for i in range(steps):
            launch(i % replicas)
        h1 = time.perf_counter()
        end.record()
        end.synchronize()
        if (h1 - h0) * 1e3 < e_spin.elapsed_time(start):
            break
        spin *= 4
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def graph_matches_eager(launch, replicas, steps=3):
    """A captured graph of `steps` launches replays to what the same last
    launch gives eagerly (returns the graph's output check)."""
    import torch

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            launch(i % replicas)
    out = launch.output
    g.replay()
    torch.cuda.synchronize()
    y_graph = out.clone()
    out.fill_(0)
    launch((steps - 1) % replicas)
    torch.cuda.synchronize()
    del g
    return bool(torch.equal(y_graph, out))


def clocks_under_load(launch, ms_per_launch):
    """GPU clocks as rocm-smi reads them while about 1.5 s of streaming-read
    launches are queued (read only, nothing set); None where rocm-smi is not
    available.  A child process, started after the launches are enqueued."""
    import re
    import shutil
    import subprocess

    import torch

    n = max(1, int(1500 / max(ms_per_launch, 1e-3)))
    for _ in range(n):
        launch()
    try:
        # rocm-smi is a Python script: run it with this interpreter rather than
        # through its `#!/usr/bin/env` line, so that the child does not replace
        # itself with another program (under a counter-collecting profiler the
        # preloaded library has already initialised the GPU in that child)
        smi = shutil.which("rocm-smi")
        if smi is None:
            raise FileNotFoundError("rocm-smi")
        r = subprocess.run([sys.executable, smi, "--showclocks", "--json"], capture_output=True, text=True,
                           timeout=30)
        card = next(iter(json.loads(r.stdout[r.stdout.index("{"):]).values()))
        mhz = {k.split()[0]: int(re.search(r"(\d+)", v).group(1)) for k, v in card.items() if "speed" in k}
    except Exception:  # no rocm-smi, or an output this parser does not know
        mhz = None
    torch.cuda.synchronize()
    return None if not mhz else {f"{k}_MHz": v for k, v in mhz.items()}


def calibrate(ngq):
    """Attainable HBM read rate (own streaming-read kernel) and a torch copy of
    known size (the reference point for the traffic counters)."""
    import torch

    out = {}
    nbytes = 4 << 30
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    ms = time_steps(lambda i: ngq.ngq_stream_read(buf, sink), 1, 10, 3)
    out["stream_read_GBps"] = nbytes / ms / 1e6
    out["clocks_under_load"] = clocks_under_load(lambda: ngq.ngq_stream_read(buf, sink), ms)
    del buf
    cb = 1 << 30
    src = torch.zeros(cb, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ms = time_steps(lambda i: dst.copy_(src), 1, 10, 3)
    out["torch_copy_bytes"] = cb
    out["torch_copy_GBps"] = 2 * cb / ms / 1e6  # read + write
    del src, dst
    torch.cuda.empty_cache()
    return out


def run_projection(ngq, w, T, steps, warmup):
    import torch

    rot = Rotation(ngq, w, T)
    y = torch.empty((T, w.N), dtype=torch.bfloat16, device="cuda")
    lib = ngq.lib()
    wp = [rot.wq[i].data_ptr() for i in range(rot.replicas)]
    sp = [rot.s[i].data_ptr() for i in range(rot.replicas)]
    xp, yp = rot.x.data_ptr(), y.data_ptr()
    bits = w.bits | (ngq.NGQ_SCALE_BF16 if w.scale_bf16 else 0)

    def launch(i):
        st = lib.ngq_gemm(T, w.K, w.N, bits, 64, xp, wp[i], sp[i], yp, torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise ngq.NgqError(st, "ngq_gemm")
    launch.output = y

    ms = time_steps(launch, rot.replicas, steps, warmup)
    return ms, rot, y, launch


def run_swiglu(ngq, T, steps, warmup):
    import torch

    import synthetic

    wgu, wdn = synthetic.WORKLOADS["gate_up"], synthetic.WORKLOADS["down"]
    n_ff = synthetic.N_FF
    rg = Rotation(ngq, wgu, T)
    rd = Rotation(ngq, wdn, T)
    h = torch.empty((T, n_ff), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T, wdn.N), dtype=torch.bfloat16, device="cuda")
    ms_gu = time_steps(lambda i: ngq.ngq_swiglu_gemm(rg.x, rg.wq[i], rg.s[i], 4, n_ff, h=h), rg.replicas, steps,
                       warmup)
    ms_dn = time_steps(lambda i: ngq.ngq_gemm(h, rd.wq[i], rd.s[i], 4, wdn.N, y=y), rd.replicas, steps, warmup)
    ws = torch.empty(ngq.ngq_splitk_workspace_bytes(wdn.K, wdn.N, 4), dtype=torch.uint8, device="cuda")
    ms_sk = time_steps(lambda i: ngq.ngq_gemm_splitk(h, rd.wq[i], rd.s[i], 4, wdn.N, y=y, workspace=ws),
                       rd.replicas, steps, warmup)
    xn = torch.empty((T, wdn.N), dtype=torch.bfloat16, device="cuda")

    def two_calls(i):
        ngq.ngq_gemm(h, rd.wq[i], rd.s[i], 4, wdn.N, y=y)
        ngq.ngq_rms_rescale(y, x=xn)

    ms_dr = time_steps(two_calls, rd.replicas, steps, warmup)
    ms_fr = time_steps(lambda i: ngq.ngq_gemm_rescale(h, rd.wq[i], rd.s[i], 4, wdn.N, y=y, x_next=xn, workspace=ws),
                       rd.replicas, steps, warmup)
    # the residual: the layer's input x (T x 5120), read once more
    ms_rr = time_steps(lambda i: ngq.ngq_gemm_residual_rescale(h, rd.wq[i], rd.s[i], 4, wdn.N, rg.x, y=y, x_next=xn,
                                                               workspace=ws), rd.replicas, steps, warmup)
    b_gu = algorithmic_bytes(ngq, wgu, T, n_out=n_ff)
    b_dn = algorithmic_bytes(ngq, wdn, T)
    b_dr = b_dn + 2 * T * wdn.N  # and the rescaled rows written
    b_rr = b_dr + 2 * T * wdn.N  # and the residual read
    del rg, rd
    torch.cuda.empty_cache()
    return [
        {"workload": "gate_up+SwiGLU int4 K=5120 N=2x17408", "T": T, "us": ms_gu * 1e3,
         "GBps": b_gu / ms_gu / 1e6, "pct_peak": 100 * b_gu / ms_gu / 1e6 / PEAK_GBS},
        {"workload": "down int4 K=17408 N=5120", "T": T, "us": ms_dn * 1e3,
         "GBps": b_dn / ms_dn / 1e6, "pct_peak": 100 * b_dn / ms_dn / 1e6 / PEAK_GBS},
        {"workload": "down int4 K=17408 N=5120, ngq_gemm_splitk (two launches)", "T": T, "us": ms_sk * 1e3,
         "GBps": b_dn / ms_sk / 1e6, "pct_peak": 100 * b_dn / ms_sk / 1e6 / PEAK_GBS},
        {"workload": "down + RMS rescale, ngq_gemm then ngq_rms_rescale", "T": T, "us": ms_dr * 1e3,
         "GBps": b_dr / ms_dr / 1e6, "pct_peak": 100 * b_dr / ms_dr / 1e6 / PEAK_GBS},
        {"workload": "down + RMS rescale, ngq_gemm_rescale (split K, fused closing kernel)", "T": T,
         "us": ms_fr * 1e3, "GBps": b_dr / ms_fr / 1e6, "pct_peak": 100 * b_dr / ms_fr / 1e6 / PEAK_GBS},
        {"workload": "down + residual + RMS rescale, ngq_gemm_residual_rescale (split K, fused closing kernel)",
         "T": T, "us": ms_rr * 1e3, "GBps": b_rr / ms_rr / 1e6, "pct_peak": 100 * b_rr / ms_rr / 1e6 / PEAK_GBS},
    ]


def run_prefill(ngq, Ts, steps):
    """Prefill-size T (token x column tiles): the QK, gate/value and down
    projections at each T, and gate/up + SwiGLU at the largest, as TFLOP/s
    against the dense bf16 MFMA peak (2 T K N flop per projection; the weights
    are reused across the tokens, so the MFMA units bound it, not HBM)."""
    import torch

    import synthetic

    out = []

    def record(label, w, T, ms, n_out):
        flop = 2.0 * T * w.K * w.N
        b = algorithmic_bytes(ngq, w, T, n_out=n_out)
        out.append({"workload": label, "T": T, "us": ms * 1e3, "TFLOPs": flop / ms / 1e9,
                    "pct_mfma_bf16_peak": 100 * flop / ms / 1e9 / PEAK_BF16_TFLOPS, "GBps": b / ms / 1e6})

    for T in Ts:
        for name in ("qk", "gv", "down"):
            w = synthetic.WORKLOADS[name]
            ms, rot, _, _ = run_projection(ngq, w, T, steps, 3)
            record(f"{name} int{w.bits} K={w.K} N={w.N}", w, T, ms, w.N)
            del rot
            torch.cuda.empty_cache()
    if Ts:
        T = max(Ts)
        w = synthetic.WORKLOADS["gate_up"]
        rot = Rotation(ngq, w, T)
        h = torch.empty((T, synthetic.N_FF), dtype=torch.bfloat16, device="cuda")
        ms = time_steps(lambda i: ngq.ngq_swiglu_gemm(rot.x, rot.wq[i], rot.s[i], 4, synthetic.N_FF, h=h),
                        rot.replicas, steps, 3)
        record("gate_up+SwiGLU int4 K=5120 N=2x17408", w, T, ms, synthetic.N_FF)
        del rot
        torch.cuda.empty_cache()
    return out


ATTAINABLE = {"qk": 32, "gv": 48, "qk8": 32}  # tile columns of the streaming pattern per workload


def run_attainable(ngq, steps):
    """The weight stream alone in the streaming kernel's access pattern
    (ngq_stream_tiles: same tiles, waves, pair order and loads; no X, no
    compute), per workload, cold: what a launch of these weight bytes can
    attain in that pattern."""
    import torch

    import synthetic

    out = {}
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    for name, cols in ATTAINABLE.items():
        w = synthetic.WORKLOADS[name]
        rot = Rotation(ngq, w, 1)
        ms = time_steps(lambda i: ngq.ngq_stream_tiles(rot.wq[i], rot.s[i], w.K, w.N, w.bits, cols, sink),
                        rot.replicas, steps, 10)
        b = packed_bytes(ngq, w) + ngq.ngq_scale_bytes(w.K, w.N, w.bits)
        out[name] = {"us": ms * 1e3, "weight_bytes": b, "GBps": b / ms / 1e6, "pct_peak": 100 * b / ms / 1e6 / PEAK_GBS,
                     "pattern": f"{cols}-column tiles, {(5 if w.bits == 8 else 10) if cols == 32 else 8} waves, "
                                "one pair in flight per wave"}
        del rot
        torch.cuda.empty_cache()
    return out


def run_tiny(ngq, steps):
    """The tiny int4 GEMV (T=1, K=256, N=256; 32 KB of weights): latency bound,
    reported in microseconds; its replicas are L2/MALL resident (labelled)."""
    import torch

    import synthetic

    w = synthetic.WORKLOADS["tiny"]
    nb = packed_bytes(ngq, w)
    wq, sc, x = synthetic.device_replicas(w, 1, steps, nb, seed=0)
    y = torch.empty((1, w.N), dtype=torch.bfloat16, device="cuda")
    ms = time_steps(lambda i: ngq.ngq_gemm(x, wq[i], sc[i], 4, w.N, y=y), steps, steps, 10)
    return {"workload": "tiny int4 GEMV T=1 K=256 N=256", "us": ms * 1e3,
            "cache": f"{steps} replicas of {nb + ngq.ngq_scale_bytes(w.K, w.N, 4)} B (cache resident: latency bound)"}


def cpu_configs(ngq, threads):
    """The oracle's CPU time per workload and T on `threads` host threads (one
    run each; random packed bytes, scales and x of the workload's shape), and
    the stacked layer (QK, gate/value, gate/up + SwiGLU, down, rescale) times
    64, labelled extrapolated."""
    import numpy as np

    import oracle
    import synthetic

    def inputs(w, T, seed):
        g = np.random.default_rng(seed)
        nb = packed_bytes(ngq, w)
        packed = synthetic.random_words(nb, g)
        scales = synthetic.draw_scales(w.K, w.N, w.scale_lo, w.scale_hi, w.scale_bf16, g)
        return synthetic.draw_x(T, w.K, g), packed, scales

    rows, layer = [], {}
    for name, Ts in (("tiny", (1,)), ("qk", (1, 2, 4, 8)), ("gv", (1, 2, 4, 8)), ("gate_up", (1, 2, 4, 8)),
                     ("down", (1, 2, 4, 8))):
        w = synthetic.WORKLOADS[name]
        x8, packed, scales = inputs(w, max(Ts), 11)
        for T in Ts:
            x = x8[:T]
            t0 = time.perf_counter()
            y64 = oracle.gemm(x, packed, scales, w.K, w.N, w.bits, w.scale_bf16, nthreads=threads)
            if name == "gate_up":
                oracle.swiglu(y64[:, :synthetic.N_FF], y64[:, synthetic.N_FF:])
            dt = time.perf_counter() - t0
            n_out = synthetic.N_FF if name == "gate_up" else w.N
            b = algorithmic_bytes(ngq, w, T, n_out=n_out)
            rows.append({"workload": name, "T": T, "us": dt * 1e6, "GBps": b / dt / 1e9})
            if name != "tiny":
                layer.setdefault(T, 0.0)
                layer[T] += dt
    # the rescale of the layer's down output (T x 5120)
    g = np.random.default_rng(12)
    stack = []
    for T, dt in sorted(layer.items()):
        z = synthetic.draw_x(T, synthetic.HIDDEN, g)
        t0 = time.perf_counter()
        oracle.rms_rescale(z)
        dt += time.perf_counter() - t0
        stack.append({"T": T, "us_per_layer": dt * 1e6, "ms_per_64_layers_extrapolated": 64 * dt * 1e3})
    return {"threads": threads, "runs": "one each", "projections": rows, "stack_64_layers_extrapolated": stack}


def summarize_trace(path):
    """Per-kernel duration percentiles of a rocprofv3 kernel-trace CSV."""
    import csv
    import statistics

    durs = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r.get("Kernel_Name", "")
            d = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            durs.setdefault(name, []).append(d / 1e3)
    out = []
    for name, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        v.sort()
        q = lambda f: v[min(len(v) - 1, int(f * (len(v) - 1) + 0.5))]
        out.append({"kernel": name[:160], "calls": len(v), "median_us": statistics.median(v), "p10_us": q(0.1),
                    "p90_us": q(0.9), "mean_us": sum(v) / len(v)})
    return out


def gpu_output(ngq, rot, y_dev):
    """Recompute replica 0 on the GPU; host copies of its inputs and output."""
    import numpy as np
    import torch

    w = rot.w
    ngq.ngq_gemm(rot.x, rot.wq[0], rot.s[0], w.bits, w.N, y=y_dev)
    torch.cuda.synchronize()
    yb = y_dev.view(torch.int16).cpu().numpy().view(np.uint16)
    packed = rot.wq[0].cpu().numpy()
    scales = rot.s[0].view(torch.int16).cpu().numpy().view(np.uint16)
    x = rot.x.view(torch.int16).cpu().numpy().view(np.uint16)
    return x, packed, scales, yb


def run_stack(ngq, layers, passes, Ts=(1, 2, 4, 8), side=True):
    """The stacked-layer sweep: `layers` layers with distinct weights (QK, gate/
    value, gate/up + SwiGLU, down, RMS rescale each), chained through the
    rescaled down output.  Timed per full pass from x0 as a captured graph with
    the three projections of x fused into one ngq_multi_gemm call and the
    down projection split over K (the reported figure), and for comparison
    eager (one library call at a time from Python, unfused), as a graph of the
    unfused calls in order, and as a graph with QK and gate/value on side
    streams.  Each graph must reproduce its own eager output bit for bit; the
    fused chain follows the unfused one up to rounding (its down projection
    groups the fp32 sums differently).  The weights far exceed the caches, so
    every pass streams them from HBM."""
    import numpy as np
    import torch

    import synthetic
    from groupwise_int_weight_amd.stack import Stack, layer_bytes

    weights = synthetic.device_stack(layers, ngq.ngq_packed_bytes, seed=0)
    out = []

    def time_graph(st, x0):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            st.forward(x0)
        g.replay()  # untimed upload
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(LEAD_CYCLES)
        e0.record()
        for _ in range(passes):
            g.replay()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) / passes, st.x.clone()

    for T in Ts:
        x0 = torch.from_numpy(synthetic.stack_x0(T).view(np.int16)).to("cuda").view(torch.bfloat16)
        st = Stack(weights, T)
        st.forward(x0)  # warm-up pass
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(passes):
            st.forward(x0)
        e1.record()
        e1.synchronize()
        eager_ms = e0.elapsed_time(e1) / passes
        eager_x = st.x.clone()
        graph_ms, gx = time_graph(st, x0)
        same = bool(torch.equal(gx, eager_x))
        fz = Stack(weights, T, fused=True)
        fz.forward(x0)
        fused_eager_x = fz.x.clone()
        fused_ms, fx = time_graph(fz, x0)
        fused_same = bool(torch.equal(fx, fused_eager_x))
        # the split-K down projection groups its sums differently: the fused
        # chain follows the unfused one up to rounding
        fused_rel = float(torch.linalg.vector_norm((fx.float() - eager_x.float())) /
                          torch.linalg.vector_norm(eager_x.float()))
        del fz
        conc_ms = None
        if side:
            conc = Stack(weights, T, concurrent=True)
            conc_ms, cx = time_graph(conc, x0)
            same = same and bool(torch.equal(cx, eager_x))
            del conc
        b = layer_bytes(T, ngq.ngq_packed_bytes) * layers
        out.append({"T": T, "layers": layers, "passes": passes,
                    "eager_us_per_layer": eager_ms * 1e3 / layers,
                    "graph_us_per_layer": fused_ms * 1e3 / layers, "graph_ms_per_pass": fused_ms,
                    "bytes_per_pass": b, "GBps": b / fused_ms / 1e6, "pct_peak": 100 * b / fused_ms / 1e6 / PEAK_GBS,
                    "graph_matches_eager": fused_same, "rel_l2_vs_unfused": fused_rel,
                    "unfused_graph_us_per_layer": graph_ms * 1e3 / layers, "unfused_graph_matches_eager": same,
                    "side_streams_graph_us_per_layer": None if conc_ms is None else conc_ms * 1e3 / layers})
        del st
    del weights
    torch.cuda.empty_cache()
    return out


HIDDEN = 5120


def run_fused(ngq, Ts, steps, sets=8):
    """The three projections of one x (QK, gate/value, gate/up + SwiGLU) as one
    ngq_multi_gemm launch, rotating over `sets` distinct weight sets (1.3 GB,
    past the caches), timed per launch in a captured graph."""
    import numpy as np
    import torch

    import synthetic
    from groupwise_int_weight_amd.stack import LAYER_PLAN, Stack

    weights = synthetic.device_stack(sets, ngq.ngq_packed_bytes, seed=1)
    out = []
    for T in Ts:
        st = Stack(weights, T)
        st.x.copy_(torch.from_numpy(synthetic.stack_x0(T).view(np.int16)).to("cuda").view(torch.bfloat16))

        def launches(k):
            for i in range(k):
                st.project(i % sets)
        launches(sets)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            launches(steps)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(LEAD_CYCLES)
        e0.record()
        g.replay()
        e1.record()
        e1.synchronize()
        ms = e0.elapsed_time(e1) / steps
        b = 0
        for name, K, N, bits, _, kind in LAYER_PLAN[:3]:
            ncols = 2 * N if kind == "swiglu" else N
            b += ngq.ngq_packed_bytes(K, ncols, bits) + (K // 64) * ncols * 2 + 2 * T * N
        b += 2 * T * HIDDEN  # x, read once
        out.append({"workload": "qk + gv + gate/up-SwiGLU in one ngq_multi_gemm", "T": T, "us": ms * 1e3,
                    "GBps": b / ms / 1e6, "pct_peak": 100 * b / ms / 1e6 / PEAK_GBS})
        del g, st
    del weights
    torch.cuda.empty_cache()
    return out


def run_valu_vs_mfma(ngq, steps, reps, Ts=(1, 2, 4, 8)):
    """The streaming pipeline with its two inner steps, forced on the same
    shapes: v_mfma (NGQ_KERNEL_STREAM) against v_dot2 on the VALU
    (NGQ_KERNEL_DOT), 32-column tiles, for int4 (QK shape), int5 (gate/value
    shape) and int8 (QK shape) at each T.  The candidates are timed
    alternately, `reps` graphs each (median reported), on the same cold
    replicas, each taking every place in the order in turn; the library's
    own choice is timed beside them.  Each
    candidate's output must match the library's within 4e-3 relative L2 (the
    two sum in different orders, so bit equality is not expected)."""
    import statistics

    import torch

    import synthetic

    rows = []
    names = {ngq.NGQ_KERNEL_STREAM: "mfma", ngq.NGQ_KERNEL_DOT: "valu"}
    for name in ("qk", "gv", "qk8"):
        w = synthetic.WORKLOADS[name]
        for T in Ts:
            rot = Rotation(ngq, w, T)
            y = torch.empty((T, w.N), dtype=torch.bfloat16, device="cuda")
            ref = ngq.ngq_gemm(rot.x, rot.wq[0], rot.s[0], w.bits, w.N).float()
            times = {p: [] for p in names}
            times[ngq.NGQ_KERNEL_AUTO] = []
            order = list(times)
            for rep in range(reps):
                # each candidate takes every place in the order in turn
                for path in order[rep % 3:] + order[:rep % 3]:
                    prev = ngq.ngq_debug_force_kernel(path)
                    try:
                        times[path].append(1e3 * time_steps(
                            lambda i: ngq.ngq_gemm(rot.x, rot.wq[i], rot.s[i], w.bits, w.N, y=y),
                            rot.replicas, steps, 5))
                    finally:
                        ngq.ngq_debug_force_kernel(prev)
            rel = {}
            for path in names:
                prev = ngq.ngq_debug_force_kernel(path)
                try:
                    out = ngq.ngq_gemm(rot.x, rot.wq[0], rot.s[0], w.bits, w.N).float()
                finally:
                    ngq.ngq_debug_force_kernel(prev)
                rel[names[path]] = float(torch.linalg.vector_norm(out - ref) / torch.linalg.vector_norm(ref))
                assert rel[names[path]] < 4e-3, (name, T, names[path], rel[names[path]])
            med = {k: statistics.median(v) for k, v in times.items()}
            b = algorithmic_bytes(ngq, w, T)
            row = {"workload": f"{name} int{w.bits} K={w.K} N={w.N}", "T": T,
                   "mfma_us": med[ngq.NGQ_KERNEL_STREAM], "valu_us": med[ngq.NGQ_KERNEL_DOT],
                   "library_us": med[ngq.NGQ_KERNEL_AUTO],
                   "faster": "valu" if med[ngq.NGQ_KERNEL_DOT] < med[ngq.NGQ_KERNEL_STREAM] else "mfma",
                   "valu_over_mfma": med[ngq.NGQ_KERNEL_DOT] / med[ngq.NGQ_KERNEL_STREAM],
                   "library_pct_peak": 100 * b / (med[ngq.NGQ_KERNEL_AUTO] * 1e3) / PEAK_GBS,
                   "rel_l2_vs_library": rel}
            rows.append(row)
            print(json.dumps(row), flush=True)
            del rot, y, ref
            torch.cuda.empty_cache()
    return rows


def host_threads() -> int:
    """The logical cores this process may run on (its CPU affinity, which a
    container's CPU share narrows), not the machine's total."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except (AttributeError, OSError):
        return max(1, os.cpu_count() or 1)


def cpu_baseline(w, T, host, bytes_full):
    """The CPU leg: the oracle as it stands timed on the host cores over the
    whole projection of replica 0, and the parity of the GPU's output for that
    replica against the oracle on sampled columns (the only place bench.py
    runs the oracle)."""
    import numpy as np

    import oracle
    from tests.parity import compare

    x, packed, scales, yb = host
    threads = host_threads()
    ncols = w.N  # the whole projection: ~2-3 s of single-core work at T=8
    cols = np.arange(ncols, dtype=np.int32)

    def run(nthreads):
        t0 = time.perf_counter()
        oracle.gemm(x, packed, scales, w.K, w.N, w.bits, w.scale_bf16, cols=cols, nthreads=nthreads)
        return time.perf_counter() - t0

    walls = [run(threads) for _ in range(3)]
    dt = sorted(walls)[1]
    dt1 = run(1)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    cpu = {
        "value": bytes_full / dt / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"one full T={T} projection ({ncols} of {w.N} columns, fp64 scalar oracle, columns split over "
                  f"{threads} threads), median of 3 runs ({', '.join(f'{v:.3f}' for v in walls)} s wall); value = "
                  f"its algorithmic bytes / wall time",
        "us_per_projection_equiv": dt * 1e6,
        "single_thread": {"value": bytes_full / dt1 / 1e9, "unit": "GB/s", "wall_s": dt1},
        "host_cpus": os.cpu_count(),
        "affinity_cpus": threads,
        "cpu_model": model,
    }
    # parity of the timed configuration: every output column
    y64, axw, axs = oracle.gemm(x, packed, scales, w.K, w.N, w.bits, w.scale_bf16, nthreads=threads,
                                with_bounds=True)
    parity = compare(yb, y64, axw, axs, w.K, w.bits)
    parity["columns_checked"] = int(w.N)
    return cpu, parity


def kernel_sha():
    """Hash of the kernel source's code: comments, trailing blanks and blank
    lines removed, so that a comment edit keeps the traffic figures taken on
    the same code."""
    import re

    with open(KERNEL_SRC) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in src.splitlines())
    return hashlib.sha256("\n".join(ln for ln in lines if ln).encode()).hexdigest()[:16]


def traffic_for(name, T):
    """HBM bytes per launch from committed counter runs, if the kernel source is
    the one they were taken on."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_sha") != kernel_sha():
        return None
    entry = d.get("workloads", {}).get(f"{name}_T{T}")
    return None if entry is None else entry.get("bytes_per_launch")


def main():
    args = parse()
    if args.summarize_trace:
        for row in summarize_trace(args.summarize_trace):
            print(json.dumps(row))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this path is not sharded "
              f"across GPUs)", file=sys.stderr)
        sys.exit(2)
    import torch

    import groupwise_int_weight_amd as ngq
    import synthetic

    assert torch.cuda.is_available(), "bench needs a HIP device"
    torch.cuda.set_device(0)
    ngq.lib()
    if args.fused:
        print(json.dumps({"fused": run_fused(ngq, (args.fused,), args.sweep_steps)}), flush=True)
        return
    if args.valu_vs_mfma:
        print(json.dumps({"valu_vs_mfma": run_valu_vs_mfma(ngq, args.sweep_steps, args.ab_reps)}), flush=True)
        return

    w = synthetic.WORKLOADS[args.workload]
    T = args.T
    ms, rot, y, launch = run_projection(ngq, w, T, args.steps, args.warmup)
    nbytes = algorithmic_bytes(ngq, w, T)
    gbps = nbytes / ms / 1e6
    # the launch replays from a captured graph to the eager result
    graph_ok = graph_matches_eager(launch, rot.replicas)
    host = gpu_output(ngq, rot, y)
    cold = rot.cold_bytes
    replicas = rot.replicas
    del rot
    torch.cuda.empty_cache()

    sweep = []
    if not args.no_sweep:
        for name in ("qk", "gv"):
            wl = synthetic.WORKLOADS[name]
            # T > 8: the verify rounds of several requests in one call
            for t in (1, 2, 4, 8, 16, 32, 64):
                ms_t, r, _, _ = run_projection(ngq, wl, t, args.sweep_steps, 10)
                b = algorithmic_bytes(ngq, wl, t)
                sweep.append({"workload": f"{name} int{wl.bits} K={wl.K} N={wl.N}", "T": t, "us": ms_t * 1e3,
                              "GBps": b / ms_t / 1e6, "pct_peak": 100 * b / ms_t / 1e6 / PEAK_GBS})
                del r
                torch.cuda.empty_cache()
        for t in (1, 8):
            sweep.extend(run_swiglu(ngq, t, args.sweep_steps, 10))
        sweep.extend(run_fused(ngq, (1, 8), args.sweep_steps))
        wl = synthetic.WORKLOADS["qk8"]  # int8: reported, not part of the metric
        for t in (1, 8):
            ms_t, r, _, _ = run_projection(ngq, wl, t, args.sweep_steps, 10)
            b = algorithmic_bytes(ngq, wl, t)
            sweep.append({"workload": f"qk-shaped int8 K={wl.K} N={wl.N}", "T": t, "us": ms_t * 1e3,
                          "GBps": b / ms_t / 1e6, "pct_peak": 100 * b / ms_t / 1e6 / PEAK_GBS})
            del r
            torch.cuda.empty_cache()

    attainable = run_attainable(ngq, args.sweep_steps)
    names_pct = {f"{n} int{synthetic.WORKLOADS[n].bits} K={synthetic.WORKLOADS[n].K} N={synthetic.WORKLOADS[n].N}": n
                 for n in ("qk", "gv")}
    names_pct["qk-shaped int8 K=5120 N=8192"] = "qk8"
    for row in sweep:
        base = names_pct.get(row["workload"])
        if base is not None and row["T"] <= 8:
            row["pct_of_attainable"] = 100 * attainable[base]["us"] / row["us"]
    tiny = run_tiny(ngq, args.sweep_steps)

    prefill = None if args.no_prefill else run_prefill(ngq, tuple(args.prefill_t), min(args.sweep_steps, 20))

    stack = None if args.no_stack else run_stack(ngq, args.stack_layers, args.stack_passes, tuple(args.stack_t),
                                                 side=not args.no_stack_side)

    # last: its 4 GiB stream and 1 GiB copies leave the next measurement slow
    calib = {} if args.no_calibration else calibrate(ngq)

    cpu, parity = (None, {"oracle": "not run (--no-cpu-baseline)"}) if args.no_cpu_baseline else \
        cpu_baseline(w, T, host, nbytes)
    if cpu is not None and not args.no_cpu_configs:
        cpu["per_workload"] = cpu_configs(ngq, host_threads())
    parity["graph_replay_matches_eager"] = graph_ok

    traffic = traffic_for(args.workload, T)
    names = {"qk": "GDN-QK-like Q4 projection", "gv": "attention gate/value-like Q5 projection"}
    line = {
        "metric": METRIC,
        "value": gbps,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": names[args.workload], "T": T, "K": w.K, "N": w.N, "bits": w.bits, "group": 64,
            "scales": "bf16" if w.scale_bf16 else "fp16", "accumulate": "fp32", "out": "bf16",
            "cache": f"cold: the {args.steps} timed launches touch {min(args.steps, replicas)} distinct weight "
                     f"replicas ({min(args.steps, replicas) * cold / replicas / 2**30:.2f} GiB; "
                     f"the 256 MB Infinity Cache holds about {256e6 / (cold / replicas):.0f})",
            "parallelism": "single GPU",
        },
        "us_per_projection": ms * 1e3,
        "pct_of_peak": 100 * gbps / PEAK_GBS,
        "pct_of_attainable": 100 * attainable[args.workload]["us"] / (ms * 1e3) if args.workload in attainable else None,
        "attainable": attainable,
        "tiny": tiny,
        "roofline": {
            "bound": "hbm",
            "achieved": gbps,
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": gbps / PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": nbytes,
        },
        "cpu_baseline": cpu,
        "calibration": calib,
        "parity": parity,
        "sweep": sweep,
        "prefill": prefill,
        "stack": stack,
        "context": {"rtx4090_single_op_us": {"attention_q5_gate_value_t8": 39.936, "gdn_qk_q4_t8": 31.744},
                    "note": "the pages' own timings on another GPU with unstated shapes; not a target"},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
