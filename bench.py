"""Throughput of the forward-convolution hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--trials T] [--mode cold|warm]
                    [--no-cpu-baseline] [--no-secondary] [--only SUBSTRING]

A step is one launch of the dense 3x3 bf16 layer (X[32,58,58,64],
F[3,3,64,64] -> Y[32,56,56,64], bf16 output, fp32 accumulation) through the C
ABI. Inputs are resident in HBM before the timed region. In the default cold
mode the steps rotate over enough distinct X/F/Y buffer sets (>= 1 GB) that
each launch reads its operands from HBM rather than from the 256 MB
memory-side cache; warm mode reuses one set. The line also carries a warm
measurement of the same layer, labelled as such.

Exactly K launches are captured into one HIP graph (torch.cuda.CUDAGraph)
and replayed once per trial, so host launch overhead does not starve a
kernel that runs for a few microseconds. Each timed region is bracketed by
synchronisations and HIP events on the stream the kernels run on; a short
spin kernel ahead of the first event keeps the host's graph submission out
of the region. The value is the median of T trials.

Prints ONE JSON line. Besides the headline it carries `secondary`: the other
workloads (1x1 bf16 and fp32, the windowed layers, the depthwise exact layer,
the depthwise sweep) measured the same way, each against its own roofline and
beside a copy of the same number of bytes.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2516.6   # dense bf16 MFMA (256 CU x 4096 FLOP/clk x 2.4 GHz)
F32_MFMA_PEAK_TFLOPS = 157.3     # dense fp32 MFMA
COLD_BYTES = 1 << 30             # rotate at least this much distinct memory in cold mode
# Measured HBM bytes per launch of the headline kernel: FETCH_SIZE and
# WRITE_SIZE per dispatch from two rocprofv3 --pmc runs, each scaled by what
# the same counter reads for the plain copy kernel of known size. The file
# records the hash of the kernel source it was taken on; once the source
# changes the figure no longer describes the kernel and is reported as null.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "dense_band_mfma_dense3x3_bf16_traffic.txt")
HEADLINE_SOURCE = os.path.join(ROOT, "convolution_forward_amd", "csrc", "dense_band_mfma.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--mode", choices=["cold", "warm"], default="cold")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--trials", type=int, default=7)
    ap.add_argument("--only", default=None,
                    help="run only the workloads whose name contains this text (for profiler runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also time the plain copy kernel (HBM bandwidth context, counter calibration)")
    return ap.parse_args()


class Runner:
    """Holds S buffer sets for one workload; times exactly `steps` launches
    per trial, cycling through the sets, from one captured graph."""

    def __init__(self, name, make_set, launch, set_bytes, mode, max_sets=None):
        import torch
        self.torch = torch
        self.name = name
        want = 1 if mode == "warm" else max(1, math.ceil(COLD_BYTES / set_bytes))
        if max_sets:
            want = min(want, max_sets)
        self.sets = [make_set(i) for i in range(want)]
        self.launch = launch
        self.kernels_per_launch = 1
        self.launches_run = 0          # every launch this runner made (eager and replayed)

    def _graph(self, n):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for k in range(n):
                self.launch(self.sets[k % len(self.sets)])
        torch.cuda.synchronize()
        return g

    def time(self, steps, warmup, trials):
        """Median ms per launch over `trials` timed regions of exactly `steps`
        launches each, after `warmup` untimed launches."""
        torch = self.torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):          # every set once, outside capture (first-launch work)
            for st in self.sets:
                self.launch(st)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.launches_run += len(self.sets)
        timed = self._graph(steps)
        if warmup > 0:
            self._graph(warmup).replay()
            self.launches_run += warmup
        torch.cuda.synchronize()
        results = []
        for _ in range(trials):
            start = torch.cuda.Event(enable_timing=True)
            end = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            torch.cuda._sleep(200_000)      # the GPU is busy while the host submits the graph
            start.record()
            timed.replay()
            end.record()
            torch.cuda.synchronize()
            results.append(start.elapsed_time(end) / steps)
        self.launches_run += trials * steps
        results.sort()
        return results[len(results) // 2]


def dense_runner(work, mode, out_dtype_name, dtype_name=None):
    import torch
    import convolution_forward_amd as cf
    import workloads as wl

    dt = dtype_name or work.dtype
    X0, F0 = wl.dense_inputs(work, dtype=dt)
    Ho, Wo = work.H - work.KH + 1, work.W - work.KW + 1
    ydt = {"bf16": torch.bfloat16, "f32": torch.float32}[out_dtype_name]
    lib = cf.load_library()
    xdt = cf.CONV_BF16 if dt == "bf16" else cf.CONV_F32
    ydc = cf.CONV_BF16 if out_dtype_name == "bf16" else cf.CONV_F32
    esz = 2 if dt == "bf16" else 4
    ysz = 2 if out_dtype_name == "bf16" else 4
    set_bytes = X0.numel() * esz + F0.numel() * esz + work.N * Ho * Wo * work.Cout * ysz

    def make_set(i):
        X = X0.to("cuda") if i == 0 else X0.to("cuda").clone()
        F = F0.to("cuda") if i == 0 else F0.to("cuda").clone()
        Y = torch.empty((work.N, Ho, Wo, work.Cout), dtype=ydt, device="cuda")
        return (X, F, Y)

    def launch(st):
        X, F, Y = st
        rc = lib.conv2d_nhwc_fwd(X.data_ptr(), None, F.data_ptr(), None, Y.data_ptr(), None, work.N, work.H, work.W,
                                 work.Cin, work.KH, work.KW, work.Cout, xdt, ydc,
                                 torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"conv2d_nhwc_fwd failed: {cf.status_str(rc)}")

    flops = 2.0 * work.N * Ho * Wo * work.Cout * work.KH * work.KW * work.Cin
    name = f"{work.name} ({dt} X, {out_dtype_name} Y)" + ("" if mode == "cold" else f" {mode}")
    return Runner(name, make_set, launch, set_bytes, mode), flops, set_bytes


def dw_runner(work, mode, exact):
    import torch
    import convolution_forward_amd as cf
    import workloads as wl

    X0, w0 = wl.depthwise_inputs(work)
    Ho = cf.out_size(work.H, work.KH, work.stride, work.pad, work.dil)
    Wo = cf.out_size(work.W, work.KW, work.stride, work.pad, work.dil)
    Cout = work.C * work.mult
    lib = cf.load_library()
    set_bytes = (X0.numel() + w0.numel() + work.N * Cout * Ho * Wo) * 4

    def make_set(i):
        X = X0.to("cuda") if i == 0 else X0.to("cuda").clone()
        w = w0.to("cuda") if i == 0 else w0.to("cuda").clone()
        Y = torch.empty((work.N, Cout, Ho, Wo), dtype=torch.float32, device="cuda")
        return (X, w, Y)

    def launch(st):
        X, w, Y = st
        rc = lib.conv_depthwise_fwd(X.data_ptr(), w.data_ptr(), None, Y.data_ptr(), work.N, work.C, work.H, work.W,
                                    work.mult, work.KH, work.KW, work.stride, work.stride, work.pad, work.pad,
                                    work.dil, work.dil, cf.CONV_DW_EXACT if exact else cf.CONV_DW_FAST,
                                    torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"conv_depthwise_fwd failed: {cf.status_str(rc)}")

    flops = 2.0 * work.N * Cout * Ho * Wo * work.KH * work.KW
    return Runner(work.name, make_set, launch, set_bytes, mode), flops, set_bytes


def im2col_route_runner(work, mode, pack_only=False):
    """The comparison route of the lecture's sections 5-7 on the same layer:
    the explicit patch matrix (library kernel), then a library GEMM
    (torch.matmul, i.e. hipBLASLt) of it with the reshaped filter. Timed with
    the packing included; pack_only times the packing alone."""
    import torch
    import convolution_forward_amd as cf
    import workloads as wl

    X0, F0 = wl.dense_inputs(work)
    Ho, Wo = work.H - work.KH + 1, work.W - work.KW + 1
    M, K = work.N * Ho * Wo, work.KH * work.KW * work.Cin
    set_bytes = (X0.numel() + F0.numel() + M * K + M * work.Cout) * 2

    def make_set(i):
        X = X0.to("cuda") if i == 0 else X0.to("cuda").clone()
        F2 = F0.to("cuda").reshape(K, work.Cout).contiguous()
        cols = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
        Y = torch.empty((M, work.Cout), dtype=torch.bfloat16, device="cuda")
        return (X, F2, cols, Y)

    def launch(st):
        X, F2, cols, Y = st
        cf.im2col_nhwc(X, work.KH, work.KW, out=cols)
        if not pack_only:
            torch.matmul(cols, F2, out=Y)

    flops = 2.0 * M * work.Cout * K
    r = Runner(work.name + (" im2col packing only" if pack_only else " im2col route"), make_set, launch, set_bytes, mode)
    r.kernels_per_launch = 1 if pack_only else 2
    return r, flops, set_bytes, M * K * 2


# Windowed layers (stride, padding, groups, 1D) measured beside the headline:
# name, X [N,H,W,Cin], (KH, KW, Cout), stride, padding, groups, dtype.
WINDOW_LAYERS = [
    ("dense3x3_bf16 same (pad 1)", (32, 56, 56, 64), (3, 3, 64), 1, 1, 1, "bf16"),
    ("dense3x3_bf16 stride 2 pad 1 -> 128 ch", (32, 56, 56, 64), (3, 3, 128), 2, 1, 1, "bf16"),
    ("grouped3x3_bf16 8 groups (pad 1)", (32, 56, 56, 128), (3, 3, 128), 1, 1, 8, "bf16"),
    ("conv1d_bf16 K3 stride 2 pad 1 (Conv1D stem, 384 ch, 3000 frames)", (8, 1, 3000, 384), (1, 3, 384), (1, 2),
     (0, 1), 1, "bf16"),
]
# Causal depthwise Conv1D: N, C, L, K (all padding before the signal), fast mode.
CAUSAL_DW = ("dw_causal_conv1d K4 (512 ch, 4096 steps)", 16, 512, 4096, 4)


def window_runner(layer, mode):
    import torch
    import convolution_forward_amd as cf
    import workloads as wl

    name, (N, H, W, C), (KH, KW, O), stride, padding, groups, dt = layer
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    X0 = wl.random_tensor((N, H, W, C), 500).to(tdt)
    F0 = (wl.random_tensor((KH, KW, C // groups, O), 501) * (1.0 / (KH * KW * C / groups) ** 0.5)).to(tdt)
    win = cf.window(stride, padding, 1, groups)
    Ho = cf.out_size_window(H, KH, win.stride_h, win.pad_top, win.pad_bottom, 1)
    Wo = cf.out_size_window(W, KW, win.stride_w, win.pad_left, win.pad_right, 1)
    esz = X0.element_size()
    set_bytes = (X0.numel() + F0.numel() + N * Ho * Wo * O) * esz

    def make_set(i):
        X = X0.to("cuda") if i == 0 else X0.to("cuda").clone()
        F = F0.to("cuda")
        Y = torch.empty((N, Ho, Wo, O), dtype=tdt, device="cuda")
        return (X, F, Y)

    def launch(st):
        X, F, Y = st
        cf.conv2d_nhwc(X, F, out=Y, stride=stride, padding=padding, groups=groups)

    flops = 2.0 * N * Ho * Wo * O * KH * KW * C / groups
    r = Runner(name, make_set, launch, set_bytes, mode)
    X, F, Y = r.sets[0]
    variant = cf.dense_variant_for(X, F, stride=stride, padding=padding, groups=groups, out=Y)
    return r, flops, set_bytes, {1: "direct", 2: "mfma_implicit_gemm"}.get(variant)


def causal_dw_runner(mode):
    import torch
    import convolution_forward_amd as cf
    import workloads as wl

    name, N, C, L, K = CAUSAL_DW
    X0 = wl.random_tensor((N, C, 1, L), 510)
    w0 = wl.random_tensor((C, 1, K), 511)
    set_bytes = (2 * X0.numel() + w0.numel()) * 4

    def make_set(i):
        X = X0.to("cuda") if i == 0 else X0.to("cuda").clone()
        return (X, w0.to("cuda"), torch.empty_like(X, device="cuda"))

    def launch(st):
        X, w, Y = st
        cf.conv_depthwise(X, w, padding=(0, 0, K - 1, 0), exact=False, out=Y)

    r = Runner(name, make_set, launch, set_bytes, mode)
    X, w, Y = r.sets[0]
    variant = cf.depthwise_variant_for(X, w, 1, (0, 0, K - 1, 0), exact=False, out=Y)
    return r, 2.0 * N * C * L * K, set_bytes, {1: "direct", 2: "lds_tiled"}.get(variant)


def copy_runner(nbytes, mode, wide=False):
    """A copy kernel moving nbytes/2 in and nbytes/2 out per launch: what the
    memory system delivers at this size and cache state. wide=False is the
    plain grid-stride copy, wide=True the one with eight 16-byte loads in
    flight per thread and write-through stores."""
    import torch
    import convolution_forward_amd as cf

    half = (int(nbytes) // 2 + 15) // 16 * 16

    def make_set(i):
        src = torch.empty(half, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        return (src, torch.empty(half, dtype=torch.uint8, device="cuda"))

    def launch(st):
        cf.copy_bytes(st[0], st[1], wide=wide)

    return Runner("copy (wide)" if wide else "copy", make_set, launch, 2 * half, mode), 2 * half


def measure(runner, steps, warmup, trials):
    ms = runner.time(steps, warmup, trials)
    # progress on stderr (the JSON line on stdout stays the only result)
    print(f"bench: {runner.name}: {ms * 1e3:.2f} us per launch, median of {trials} trials of {steps} launches "
          f"({runner.launches_run * runner.kernels_per_launch} kernel dispatches)", file=sys.stderr, flush=True)
    return ms, steps


def copy_context(nbytes, mode, steps, warmup, trials):
    """ms per launch of the plain and the wide copy of the same byte count."""
    import torch
    out = {}
    for wide in (False, True):
        r, _ = copy_runner(nbytes, mode, wide)
        out["wide" if wide else "plain"], _ = measure(r, steps, warmup, trials)
        del r
        torch.cuda.empty_cache()
    return out


def measured_traffic():
    """HBM bytes per launch from the committed counter summary, or None when
    it is missing or was taken on a different kernel source."""
    import hashlib
    try:
        fields = {}
        with open(TRAFFIC_FILE) as f:
            for ln in f:
                if ":" in ln and not ln.startswith("#"):
                    k, v = ln.split(":", 1)
                    fields[k.strip()] = v.strip()
        with open(HEADLINE_SOURCE, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
        if fields.get("kernel_source_sha256") != sha:
            return None
        return float(fields["traffic_bytes_per_dispatch"])
    except (OSError, KeyError, ValueError):
        return None


# Single-thread AVX2 fast-mode GFLOP/s that the "Depthwise convolution" page
# ("Measured") lists for MobileNetV3-large layers after its phase-plane
# rewrite, quoted as CPU context next to the GPU lines (one image; the batch
# is not stated there). Keys are the workloads' layer shapes.
PAGES_AVX2_GFLOPS = {
    "dw_c72_5x5s2_56_exact": 38.0,
    "dw_c16_3x3s1_112": 41.0,
    "dw_c64_3x3s2_112": 18.5,       # the page gives 17-20
    "dw_c120_5x5s1_28": 50.0,
    "dw_c672_5x5s2_14": 9.0,
    "dw_c960_5x5s1_7": 13.0,
}


def _time_for(fn, budget_s, max_reps=1000):
    """Run fn repeatedly for about budget_s seconds; (passes, seconds)."""
    reps, dt = 0, 0.0
    while dt < budget_s and reps < max_reps:
        t0 = time.perf_counter()
        fn()
        dt += time.perf_counter() - t0
        reps += 1
    return reps, dt


def cpu_baseline(work):
    """The oracle, untuned, on bounded samples of the headline workload (all
    host threads and one thread) and of the depthwise exact layer (both
    thread counts), about 25 s of CPU work in all."""
    import numpy as np
    import oracle
    import workloads as wl

    threads = oracle.default_threads()
    X, F = wl.dense_inputs(work)
    Xf = X.float().numpy()
    Ff = F.float().numpy()
    Ho, Wo = work.H - work.KH + 1, work.W - work.KW + 1
    per_img = 2.0 * Ho * Wo * work.Cout * work.KH * work.KW * work.Cin

    def dense_rate(nthreads, budget):
        t0 = time.perf_counter()
        oracle.conv2d_nhwc(Xf[:1], Ff, threads=nthreads)
        t1 = time.perf_counter() - t0
        n_img = int(min(work.N, max(1, (budget / 2) // max(t1, 1e-3))))
        Xs = np.ascontiguousarray(Xf[:n_img])
        reps, dt = _time_for(lambda: oracle.conv2d_nhwc(Xs, Ff, threads=nthreads), budget)
        return reps * n_img * per_img / dt, n_img, reps, dt

    v, n_img, reps, dt = dense_rate(threads, 10.0)
    out = {"value": v / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": f"first {n_img} of {work.N} images of {work.name}, {reps} pass(es) "
                     f"(fp64-accumulate seven-loop C oracle, OpenMP {threads} threads), {dt:.1f} s"}
    v1, n1, reps1, dt1 = dense_rate(1, 5.0)
    out["single_thread"] = {"value": v1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                            "sample": f"first {n1} image(s) of {work.name}, {reps1} pass(es), {dt1:.1f} s"}
    out["host_cpu_count"] = os.cpu_count()
    out["omp_num_threads"] = os.environ.get("OMP_NUM_THREADS")

    dw = wl.DW_5X5S2_EXACT
    Xd, wd = wl.depthwise_inputs(dw)
    Xd, wd = Xd.numpy(), wd.numpy()
    Ho_d = oracle.out_size(dw.H, dw.KH, dw.stride, dw.pad, dw.dil)
    Wo_d = oracle.out_size(dw.W, dw.KW, dw.stride, dw.pad, dw.dil)
    fl_d = 2.0 * dw.N * dw.C * dw.mult * Ho_d * Wo_d * dw.KH * dw.KW
    dwo = {}
    for label, nthreads in (("all_threads", threads), ("single_thread", 1)):
        reps, dt = _time_for(lambda: oracle.depthwise_nchw(Xd, wd, stride=dw.stride, padding=dw.pad,
                                                           dilation=dw.dil, mode="exact", threads=nthreads), 3.0)
        dwo[label] = {"GFLOP/s": round(reps * fl_d / dt / 1e9, 3), "cores": nthreads, "passes": reps,
                      "seconds": round(dt, 2)}
    dwo["workload"] = dw.name + " (whole batch, exact mode: per-output fp32 loop in the pages' order)"
    dwo["pages_single_thread_avx2_GFLOP/s"] = PAGES_AVX2_GFLOPS[dw.name]
    out["depthwise_exact"] = dwo
    return out


def dense_line(name, ms, n, flops, nbytes, peak, kernel=None, copies=None):
    tf = flops / (ms * 1e-3) / 1e12
    gb = nbytes / (ms * 1e-3) / 1e9
    d = {"workload": name, "ms": ms, "launches": n, "TFLOP/s": round(tf, 2), "GB/s": round(gb, 1),
         "frac_hbm": round(gb / HBM_PEAK_GBS, 4), "frac_mfma_peak": round(tf / peak, 4), "mfma_peak": peak,
         "attainable_TFLOP/s": round(min(peak, flops / nbytes * HBM_PEAK_GBS / 1e3), 1)}
    d["frac_attainable"] = round(tf / d["attainable_TFLOP/s"], 4)
    if kernel:
        d["kernel"] = kernel
    if copies:
        d["copy_same_bytes_ms"] = copies["plain"]
        d["copy_wide_same_bytes_ms"] = copies["wide"]
        d["over_wide_copy"] = round(ms / copies["wide"], 3)
    return d


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this build runs on a single "
              "MI355X and has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch
    import convolution_forward_amd as cf
    import workloads as wl

    cf.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    want = (lambda name: args.only is None or args.only in name)
    steps, warmup, trials = args.steps, args.warmup, args.trials
    steps2 = max(200, steps // 4)

    work = wl.DENSE_3X3_BF16
    Ho, Wo = work.H - work.KH + 1, work.W - work.KW + 1
    flops = 2.0 * work.N * Ho * Wo * work.Cout * work.KH * work.KW * work.Cin
    line = {
        "metric": "conv fwd TFLOP/s (dense) and GB/s (depthwise), % of MI355X roofline",
        "value": None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "trials": trials,
        "ms_per_step": None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "dense3x3_bf16: NHWC X[32,58,58,64] bf16 * F[3,3,64,64] bf16 -> Y[32,56,56,64] bf16, "
                               "fp32 accumulate, stride 1, no padding",
                   "N": work.N, "H": work.H, "W": work.W, "Cin": work.Cin, "K": work.KH, "Cout": work.Cout,
                   "out_dtype": "bf16", "cache_mode": args.mode, "buffer_sets": None, "kernel_variant": None,
                   "timing": f"median of {trials} trials, each exactly {steps} launches replayed from one HIP graph"},
    }
    if want(work.name):
        runner, _, set_bytes = dense_runner(work, args.mode, "bf16")
        X, F, Y = runner.sets[0]
        variant = cf.dense_variant_for(X, F, out=Y)
        ms, _ = measure(runner, steps, warmup, trials)
        line["config"]["buffer_sets"] = len(runner.sets)
        del runner
        torch.cuda.empty_cache()
        tflops = flops / (ms * 1e-3) / 1e12
        gbs = set_bytes / (ms * 1e-3) / 1e9
        line["value"] = round(tflops, 2)
        line["ms_per_step"] = ms
        line["config"]["kernel_variant"] = {1: "direct", 2: "mfma_implicit_gemm"}.get(variant)
        line["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                            "algorithmic_bytes": set_bytes, "kernel_ms": ms,
                            "mfma_tflops": round(tflops, 2), "mfma_peak": BF16_MFMA_PEAK_TFLOPS,
                            "mfma_frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4)}
        # Context for the HBM fraction: copies of the same number of bytes,
        # in the same cache state, are what the memory system delivers at
        # this size (the wide copy is the faster of the two).
        cp = copy_context(set_bytes, args.mode, steps, warmup, trials)
        line["roofline"]["copy_same_bytes_ms"] = cp["plain"]
        line["roofline"]["copy_same_bytes_GBps"] = round(set_bytes / (cp["plain"] * 1e-3) / 1e9, 1)
        line["roofline"]["copy_wide_same_bytes_ms"] = cp["wide"]
        line["roofline"]["copy_wide_same_bytes_GBps"] = round(set_bytes / (cp["wide"] * 1e-3) / 1e9, 1)
        line["roofline"]["frac_of_copy"] = round(min(cp["plain"], cp["wide"]) / ms, 4)
        # The same layer with one buffer set: operands stay in the 256 MB
        # memory-side cache between launches. Labelled; not the headline.
        other = "warm" if args.mode == "cold" else "cold"
        r, _, _ = dense_runner(work, other, "bf16")
        m_o, _ = measure(r, steps, warmup, trials)
        del r
        torch.cuda.empty_cache()
        line[other] = {"label": ("one buffer set reused: X, F and Y stay in the 256 MB memory-side cache between "
                                 "launches" if other == "warm" else
                                 ">= 1 GB of distinct buffer sets rotated: every launch reads from HBM"),
                       "ms": m_o, "TFLOP/s": round(flops / (m_o * 1e-3) / 1e12, 2),
                       "GB/s": round(set_bytes / (m_o * 1e-3) / 1e9, 1),
                       "frac_mfma_peak": round(flops / (m_o * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)}

    secondary = []
    if not args.no_secondary:
        for name, make, peak in [
            ("dense1x1_bf16 (Y bf16)", lambda: dense_runner(wl.DENSE_1X1_BF16, args.mode, "bf16"),
             BF16_MFMA_PEAK_TFLOPS),
            ("dense1x1_f32", lambda: dense_runner(wl.DENSE_1X1_BF16, args.mode, "f32", "f32"), F32_MFMA_PEAK_TFLOPS),
            ("dense3x3_bf16 (Y f32)", lambda: dense_runner(wl.DENSE_3X3_BF16, args.mode, "f32"),
             BF16_MFMA_PEAK_TFLOPS),
        ]:
            if not want(name):
                continue
            r, fl, by = make()
            m, n = measure(r, steps2, warmup, trials)
            del r
            torch.cuda.empty_cache()
            cp = copy_context(by, args.mode, steps2, warmup, trials)
            secondary.append(dense_line(name, m, n, fl, by, peak, copies=cp))
            if name == "dense1x1_f32":
                # fp32 operands on the bf16 matrix cores: three bf16 parts per
                # value, six part products per fp32 product.
                tf = fl / (m * 1e-3) / 1e12
                secondary[-1]["path"] = "bf16 matrix cores, fp32 values split into three bf16 parts, six products"
                secondary[-1]["split_peak_TFLOP/s"] = round(BF16_MFMA_PEAK_TFLOPS / 6, 1)
                secondary[-1]["frac_split_peak"] = round(tf / (BF16_MFMA_PEAK_TFLOPS / 6), 4)
        if want("im2col"):
            # The explicit im2col route on the headline layer (packing included).
            r, fl, by, cols_bytes = im2col_route_runner(wl.DENSE_3X3_BF16, args.mode)
            m_route, n = measure(r, steps2, warmup, trials)
            del r
            torch.cuda.empty_cache()
            r, _, _, _ = im2col_route_runner(wl.DENSE_3X3_BF16, args.mode, pack_only=True)
            m_pack, _ = measure(r, steps2, warmup, trials)
            del r
            torch.cuda.empty_cache()
            secondary.append({"workload": "dense3x3_bf16 via explicit im2col + library GEMM (comparison route)",
                              "ms": m_route, "ms_packing": m_pack, "launches": n,
                              "TFLOP/s": round(fl / (m_route * 1e-3) / 1e12, 2),
                              "patch_matrix_bytes": cols_bytes,
                              "implicit_gemm_ms": line["ms_per_step"],
                              "route_over_implicit": (round(m_route / line["ms_per_step"], 2)
                                                      if line["ms_per_step"] else None)})
        for layer in WINDOW_LAYERS:
            if not want(layer[0]):
                continue
            r, fl, by, kv = window_runner(layer, args.mode)
            m, n = measure(r, max(100, steps2 // 2), warmup, trials)
            del r
            torch.cuda.empty_cache()
            cp = copy_context(by, args.mode, max(100, steps2 // 2), warmup, trials)
            secondary.append(dense_line(layer[0], m, n, fl, by, BF16_MFMA_PEAK_TFLOPS, kernel=kv, copies=cp))
        if want(CAUSAL_DW[0]):
            r, fl, by, kv = causal_dw_runner(args.mode)
            m, n = measure(r, steps2, warmup, trials)
            del r
            torch.cuda.empty_cache()
            cp = copy_context(by, args.mode, steps2, warmup, trials)
            gb = by / (m * 1e-3) / 1e9
            secondary.append({"workload": CAUSAL_DW[0], "kernel": kv, "ms": m, "launches": n, "GB/s": round(gb, 1),
                              "frac_hbm": round(gb / HBM_PEAK_GBS, 4), "GFLOP/s": round(fl / (m * 1e-3) / 1e9, 1),
                              "copy_same_bytes_ms": cp["plain"], "copy_wide_same_bytes_ms": cp["wide"],
                              "over_wide_copy": round(m / cp["wide"], 3)})
        for work_dw, exact in [(wl.DW_5X5S2_EXACT, True)] + [(l, False) for l in wl.DW_SWEEP]:
            if not want(work_dw.name):
                continue
            r, fl, by = dw_runner(work_dw, args.mode, exact)
            m, n = measure(r, steps2, warmup, trials)
            del r
            torch.cuda.empty_cache()
            cp = copy_context(by, args.mode, steps2, warmup, trials)
            gb = by / (m * 1e-3) / 1e9
            secondary.append({"workload": work_dw.name + (" exact" if exact else " fast"), "ms": m, "launches": n,
                              "GB/s": round(gb, 1), "frac_hbm": round(gb / HBM_PEAK_GBS, 4),
                              "GFLOP/s": round(fl / (m * 1e-3) / 1e9, 1),
                              "copy_same_bytes_ms": cp["plain"], "copy_wide_same_bytes_ms": cp["wide"],
                              "over_wide_copy": round(m / cp["wide"], 3),
                              "pages_single_thread_avx2_GFLOP/s": PAGES_AVX2_GFLOPS.get(work_dw.name)})
    line["secondary"] = secondary

    if args.copy_calibration:
        nbytes = 256 << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        for _ in range(3):
            cf.copy_bytes(src, dst)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        start.record()
        for _ in range(reps):
            cf.copy_bytes(src, dst)
        end.record()
        torch.cuda.synchronize()
        ms_copy = start.elapsed_time(end) / reps
        line["copy_calibration"] = {"bytes_read": nbytes, "bytes_written": nbytes, "ms": ms_copy,
                                    "GB/s (read+write)": round(2 * nbytes / (ms_copy * 1e-3) / 1e9, 1)}
        del src, dst

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(work)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
