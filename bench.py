"""Benchmark of the W4A16 hot path on one MI355X.

Headline (`value`): ROCmFP4 Dual 4096 x 4096, M = 1 (a decode GEMV), in GB/s of weight + scale bytes.
The same JSON line carries every other workload, each with its own roofline fraction:
  * NVFP4 2048 x 2048, M = 1;
  * the 4B-class decode sweep (36 layers x q, k, v, o, gate, up, down; NVFP4, M = 1), grouped launches
    and one launch per matrix;
  * speculative verify / small batch: gate 9728 x 2560 and down 2560 x 9728 at M = 1, 9, 16 in NVFP4,
    Dual and FAST (M = 9 is one token plus eight n-gram drafts);
  * the prefill GEMM, M = 2048, K = 4096, N = 14336, in FAST and NVFP4 (TFLOP/s), and the same matrix at
    M = 128, 256, 512; beside it, as context, the ROCm BLAS library's plain bf16 product of the same shape
    (a linear layer's y = x W^T, no dequantization), timed eagerly;
  * a plain streaming read of the same byte counts (the ceiling launch cost and memory latency leave);
  * context: the M = 1 GEMV on two large matrices (a 70B-class gate/up projection 28672 x 8192 and its down
    projection 8192 x 28672, NVFP4 and Dual, 132 MB each), where launch cost and latency are amortised, with
    a plain read of the same bytes beside each.

A step of a GEMV workload is one launch over one packed matrix. Weights are drawn by `synth`, packed on
the GPU by the library's own packers and replicated into distinct copies totalling >= 1 GiB, so every
launch reads its matrix from HBM, not from the 256 MB last-level cache. Launch i reads copy i % copies.

Timing protocol (per workload): K timed steps are captured in HIP graphs (one graph of min(K, copies)
launches, replayed, plus one for the remainder); every graph is replayed during warm-up before any
timing. Each of R repetitions replays an untimed filler graph (the other copies, so that the timed
copies are cold and the GPU queue is never empty at the start event), then the timed graphs between two
HIP events on torch's current stream (the stream the graphs launch on). Reported: the median per-step
time over the R repetitions, min, max, max/min and the raw samples. (The shader clock is not sampled here:
the SMU metrics table read through amdsmi does not follow the load on these boards; the counter-based
clock, GRBM_GUI_ACTIVE over the traced kernel time, is recorded with the rocprofv3 summaries.)

The CPU baseline (`cpu_baseline`) times the oracle (exact dequantisation + FP64 product) on a bounded
row sample of each workload, packed by the oracle's own packers, on every core of this process's
affinity mask, and compares the GPU output on the same rows with it: a workload whose sample fails that
check is reported with "parity": false and no throughput.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--reps R] [--only NAME[,NAME...]]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
COLD_BYTES = 1 << 30            # 4x the 256 MB last-level cache
BLOCK_BYTES = {"rocmfp4_dual": 18, "rocmfp4_fast": 17, "q4_0": 18}
HEADLINE = "rocmfp4_dual_4096x4096_m1"

# One-matrix GEMV workloads: name -> (synth workload id, matrix index, fmt, M)
WORKLOADS = {
    "rocmfp4_dual_4096x4096_m1": (1, 0, "rocmfp4_dual", 1),
    "nvfp4_2048x2048_m1": (0, 0, "nvfp4", 1),
    "q4_0_4096x4096_m1": (1, 0, "q4_0", 1),          # the Dual matrix in stock Q4_0 (same bytes)
}
SPEC_FMTS = ("nvfp4", "rocmfp4_dual", "rocmfp4_fast")
SPEC_SHAPES = (("gate_9728x2560", 0), ("down_2560x9728", 1))
SPEC_MS = (1, 9, 16)
for _f in SPEC_FMTS + ("q4_0",):
    for _shape, _mat in SPEC_SHAPES:
        for _m in SPEC_MS:
            WORKLOADS[f"{_f}_{_shape}_m{_m}"] = (3, _mat, _f, _m)

SECTIONS = ("headline", "nvfp4_2048", "spec", "gemm", "gemm_small", "sweep", "read_probe", "packers", "gemv_large")
# M = 1 GEMV context on large matrices: (N, K); weights N(0, 0.02) drawn on the GPU (synth.device_weights)
LARGE_SHAPES = ((28672, 8192), (8192, 28672))
LARGE_FMTS = ("nvfp4", "rocmfp4_dual")
LARGE_CFG = 5


def algorithmic_bytes(fmt: str, n: int, k: int) -> int:
    """Weight + scale bytes one product must read once (NVFP4 and Dual 0.5625 B/weight, FAST 0.53125)."""
    if fmt == "nvfp4":
        return n * (k // 2 + k // 16)
    return n * (k // 32) * BLOCK_BYTES[fmt]


def kernel_source_hash(name: str) -> str:
    path = os.path.join(ROOT, "block_scaled_fp4_w4a16_amd", "csrc", name)
    h = hashlib.sha256()
    for p in (path, os.path.join(ROOT, "block_scaled_fp4_w4a16_amd", "csrc", "common.h")):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_file: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 counters, if taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    entry = data.get(workload)
    if not entry or entry.get("source_hash") != kernel_source_hash(kernel_file):
        return None
    return entry.get("bytes_per_launch")


def host_threads() -> int:
    """Host cores this process may run on (its affinity mask)."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return max(1, os.cpu_count() or 1)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ----------------------------------------------------------------------------------------------
class Probes:
    """The benchmark's measurement kernel (libfp4probe.so): a plain streaming read."""

    def __init__(self, torch):
        path = os.path.join(ROOT, "block_scaled_fp4_w4a16_amd", "libfp4probe.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with block_scaled_fp4_w4a16_amd/build.py")
        self.torch = torch
        self.lib = ctypes.CDLL(path)
        self.lib.fp4probe_read.restype = ctypes.c_int
        self.lib.fp4probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
        self.sink = torch.zeros(256, dtype=torch.int32, device="cuda")

    def read(self, ptr: int, nbytes: int):
        rc = self.lib.fp4probe_read(ptr, nbytes, self.sink.data_ptr(), self.torch.cuda.current_stream().cuda_stream)
        if rc:
            raise RuntimeError(f"read probe launch failed ({rc})")


def graph_of(torch, fn, launches):
    """Capture fn(i) for i in `launches` into one HIP graph (the library launches on the capture stream)."""
    launches = list(launches)
    if not launches:
        return None
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(launches[0])  # warm the host code path outside capture once
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in launches:
            fn(i)
    torch.cuda.synchronize()
    return g


def time_steps(torch, fn, copies: int, steps: int, warmup: int, reps: int, probes=None, filler: int | None = None):
    """Time `steps` launches fn(i) (launch i reads copy i % copies) `reps` times; see the module docstring.

    Returns per-step seconds (median, min, max, samples) and the graph shape."""
    L = max(1, min(steps, copies))
    q, r = divmod(steps, L)
    g_main = graph_of(torch, fn, range(L))
    g_rem = graph_of(torch, fn, range(r))
    fill = range(L, copies) if L < copies else range(filler if filler is not None else copies)
    g_fill = graph_of(torch, fn, fill)
    graphs = [g for g in (g_fill, g_main, g_rem) if g is not None]
    per_round = len(fill) + L + r
    done = 0
    while done < max(warmup, 1):
        for g in graphs:
            g.replay()
        done += per_round
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    samples = []
    for _ in range(reps):
        if g_fill is not None:
            g_fill.replay()
        start.record()
        for _ in range(q):
            g_main.replay()
        if g_rem is not None:
            g_rem.replay()
        end.record()
        torch.cuda.synchronize()
        samples.append(start.elapsed_time(end) / 1e3 / steps)
    med = float(np.median(samples))
    return dict(median_s=med, min_s=float(min(samples)), max_s=float(max(samples)), samples_s=samples,
                launches_per_graph=L,
                graph_replays_per_rep=q + (1 if r else 0), reps=reps, steps=steps)


def timing_fields(t: dict) -> dict:
    return {"us_median": round(t["median_s"] * 1e6, 3), "us_min": round(t["min_s"] * 1e6, 3),
            "us_max": round(t["max_s"] * 1e6, 3), "spread": round(t["max_s"] / t["min_s"], 4),
            "samples_us": [round(v * 1e6, 3) for v in t["samples_s"]], "reps": t["reps"],
            "steps_per_rep": t["steps"], "launches_per_graph": t["launches_per_graph"]}


def hbm_roofline(nbytes: int, t: dict, traffic=None) -> dict:
    gbs = nbytes / t["median_s"] / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic}


# ----------------------------------------------------------------------------------------------
def pack_on_gpu(fp4, torch, fmt: str, w_np: np.ndarray):
    """synth fp32 weights -> the library's device packer -> kernel layout (no oracle)."""
    w = torch.from_numpy(w_np).cuda()
    pw = fp4.PackedWeight.quantize(fmt, w)
    del w
    return pw


def bench_gemv(fp4, torch, synth, name: str, steps: int, warmup: int, reps: int, probes):
    cfg, mat, fmt, m = WORKLOADS[name]
    n, k = synth.WORKLOADS[cfg]["shapes"][mat]
    w_np = synth.workload_weights(cfg, mat)
    pw = pack_on_gpu(fp4, torch, fmt, w_np)
    plane_bytes = pw.q.numel() + pw.s.numel()
    copies = max(2, -(-COLD_BYTES // plane_bytes))
    qs = [pw.q] + [pw.q.clone() for _ in range(copies - 1)]
    ss = [pw.s] + [pw.s.clone() for _ in range(copies - 1)]
    x_bits = synth.workload_activations(cfg, mat, m)
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).cuda()
    ys = [torch.empty((m, n), dtype=torch.float32, device="cuda") for _ in range(min(copies, 8))]

    def launch(i):
        fp4.w4a16_gemv(fmt, m, n, k, qs[i % copies], ss[i % copies], pw.global_scale, x, ys[i % len(ys)])

    t = time_steps(torch, launch, copies, steps, warmup, reps, probes)
    y0 = torch.empty((m, n), dtype=torch.float32, device="cuda")
    fp4.w4a16_gemv(fmt, m, n, k, qs[0], ss[0], pw.global_scale, x, y0)
    torch.cuda.synchronize()
    del qs, ss
    return dict(name=name, fmt=fmt, n=n, k=k, m=m, copies=copies, bytes=algorithmic_bytes(fmt, n, k), t=t,
                y=y0.cpu().numpy(), x_bits=x_bits, w_np=w_np, global_scale=pw.global_scale)


def bench_gemv_large(fp4, torch, synth, fmt: str, n: int, k: int, steps: int, warmup: int, reps: int, probes):
    """M = 1 GEMV on a large matrix (context: launch cost amortised), with a plain read of the same bytes."""
    mat = n + k
    w = synth.device_weights(n, k, cfg=LARGE_CFG, mat=mat)
    pw = fp4.PackedWeight.quantize(fmt, w)
    del w
    plane_bytes = pw.q.numel() + pw.s.numel()
    copies = max(2, -(-COLD_BYTES // plane_bytes))
    qs = [pw.q] + [pw.q.clone() for _ in range(copies - 1)]
    ss = [pw.s] + [pw.s.clone() for _ in range(copies - 1)]
    x_bits = synth.activations(1, k, cfg=LARGE_CFG, mat=mat)
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).cuda()
    ys = [torch.empty((1, n), dtype=torch.float32, device="cuda") for _ in range(min(copies, 8))]

    def launch(i):
        fp4.w4a16_gemv(fmt, 1, n, k, qs[i % copies], ss[i % copies], pw.global_scale, x, ys[i % len(ys)])

    t = time_steps(torch, launch, copies, steps, warmup, reps, probes)
    y0 = torch.empty((1, n), dtype=torch.float32, device="cuda")
    fp4.w4a16_gemv(fmt, 1, n, k, qs[0], ss[0], pw.global_scale, x, y0)
    torch.cuda.synchronize()
    del qs, ss, pw
    torch.cuda.empty_cache()
    nbytes = algorithmic_bytes(fmt, n, k)
    tr = bench_read_probe(torch, probes, nbytes, steps, warmup, reps)
    return dict(name=f"{fmt}_{n}x{k}_m1", fmt=fmt, n=n, k=k, m=1, mat=mat, copies=copies, bytes=nbytes, t=t,
                t_read=tr, y=y0.cpu().numpy(), x_bits=x_bits)


def bench_gemm(fp4, torch, synth, fmt: str, m: int, steps: int, warmup: int, reps: int, probes, pw=None, cfg=4,
               mat=0):
    n, k = synth.WORKLOADS[cfg]["shapes"][mat]
    if pw is None:
        pw = pack_on_gpu(fp4, torch, fmt, synth.workload_weights(cfg, mat))
    x_bits = synth.workload_activations(cfg, mat, m)
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).cuda()
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")

    def launch(_):
        fp4.w4a16_gemm(fmt, m, n, k, pw.q, pw.s, pw.global_scale, x, y)

    # the weights and x stay resident in the last-level cache between launches (one copy): the product
    # is bound by the matrix cores, not by reading them
    t = time_steps(torch, launch, steps, steps, warmup, reps, probes, filler=min(steps, 20))
    fp4.w4a16_gemm(fmt, m, n, k, pw.q, pw.s, pw.global_scale, x, y)
    torch.cuda.synchronize()
    flops = 2.0 * m * n * k
    return dict(fmt=fmt, m=m, n=n, k=k, t=t, tflops=flops / t["median_s"] / 1e12, pw=pw, x_bits=x_bits,
                y=y.cpu().numpy(), ws_bytes=fp4.w4a16_gemm_workspace_bytes(fmt, m, n, k))


def bench_dense_bf16_gemm(torch, m: int, n: int, k: int, steps: int, warmup: int, reps: int):
    """Context for the GEMM: y = x W^T of the same shape on plain bf16 weights stored N x K, as a linear
    layer holds them (torch.nn.functional.linear, i.e. the ROCm BLAS library; no dequantization, bf16
    output), timed eagerly with events around `steps` back-to-back launches."""
    import torch.nn.functional as tnf
    g = torch.Generator(device="cuda")
    g.manual_seed(4)
    x = torch.randn((m, k), generator=g, device="cuda").to(torch.bfloat16)
    w = (torch.randn((n, k), generator=g, device="cuda") * 0.02).to(torch.bfloat16)  # N x K, contiguous
    y = tnf.linear(x, w)
    for _ in range(warmup):
        y = tnf.linear(x, w)
    torch.cuda.synchronize()
    samples = []
    for _ in range(reps):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(steps):
            y = tnf.linear(x, w)
        end.record()
        torch.cuda.synchronize()
        samples.append(start.elapsed_time(end) / 1e3 / steps)
    del x, w, y
    torch.cuda.empty_cache()
    med = float(np.median(samples))
    return dict(median_s=med, min_s=float(min(samples)), max_s=float(max(samples)), samples_s=samples,
                launches_per_graph=0, graph_replays_per_rep=0, reps=reps, steps=steps)


def bench_read_probe(torch, probes, nbytes: int, steps: int, warmup: int, reps: int):
    """The plain streaming read of `nbytes` per launch over >= 1 GiB of distinct slices."""
    slot = -(-nbytes // 256) * 256
    copies = max(2, -(-COLD_BYTES // slot))
    buf = torch.empty(copies * slot, dtype=torch.uint8, device="cuda")
    buf.random_(0, 256)
    base = buf.data_ptr()

    def launch(i):
        probes.read(base + (i % copies) * slot, nbytes)

    t = time_steps(torch, launch, copies, steps, warmup, reps, probes)
    del buf
    return t


def bench_decode_sweep(fp4, torch, synth, steps: int, warmup: int, reps: int, probes):
    """The 4B-class decode sweep: 36 layers x {q, k, v, o, gate, up, down}, NVFP4, M = 1.

    Weights are N(0, 0.02) drawn on the GPU (synth.device_weights) and packed by the library's NVFP4
    packer; all 252 matrices (2.04 GB) stay resident, so each sweep streams them from HBM. A sweep is
    launched per layer the way a decoder consumes it: one grouped launch for q|k|v (same x), one for
    o, one grouped launch for gate|up (same x), one for down -- 144 launches. The same sweep with one
    launch per matrix (252 launches), and a plain streaming read with the 144 grouped launches' byte
    counts over the same 2.04 GB, are timed beside it.
    """
    cfg = 2
    layer = synth.DECODE_4B_LAYER
    mats, total_bytes = [], 0
    for li in range(36):
        row = []
        for pi, (_, n, k) in enumerate(layer):
            w = synth.device_weights(n, k, cfg=cfg, mat=7 * li + pi)
            pw = fp4.PackedWeight.quantize("nvfp4", w)
            del w
            row.append(pw)
            total_bytes += algorithmic_bytes("nvfp4", n, k)
        mats.append(row)
    torch.cuda.synchronize()

    def xb(k, mat):
        return synth.activations(1, k, cfg=cfg, mat=mat)

    x_host = [dict(attn=xb(2560, 4 * li), o=xb(4096, 4 * li + 1), mlp=xb(2560, 4 * li + 2), down=xb(9728, 4 * li + 3))
              for li in range(36)]
    xs = [{key: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).cuda() for key, v in d.items()}
          for d in x_host]
    ys = [[torch.empty((1, n), dtype=torch.float32, device="cuda") for (_, n, _) in layer] for _ in range(36)]
    which_x = ("attn", "attn", "attn", "o", "mlp", "mlp", "down")

    def item(li, pi):
        pw = mats[li][pi]
        return (pw.q, pw.s, pw.global_scale, xs[li][which_x[pi]], ys[li][pi], pw.N, pw.K)

    groups = ((0, 1, 2), (3,), (4, 5), (6,))

    def sweep_grouped(_):
        for li in range(36):
            for grp in groups:
                fp4.w4a16_gemv_batched("nvfp4", 1, [item(li, pi) for pi in grp])

    def sweep_single(_):
        for li in range(36):
            for pi in range(7):
                q, s_, g, x, y, n, k = item(li, pi)
                fp4.w4a16_gemv("nvfp4", 1, n, k, q, s_, g, x, y)

    # the 252 products as a device list: launches of up to 32 matrices each, in layer order (the
    # benchmark's products are independent, so they may share a launch; a decoder's layers could not)
    flat = [(li, pi) for li in range(36) for pi in range(7)]
    lists = [flat[i:i + 32] for i in range(0, len(flat), 32)]

    def sweep_list(_):
        for lst in lists:
            fp4.w4a16_gemv_batched("nvfp4", 1, [item(li, pi) for (li, pi) in lst])

    out = dict(bytes=total_bytes, list_launches=len(lists))
    for name, fn in (("grouped", sweep_grouped), ("single", sweep_single), ("device_list", sweep_list)):
        out[name] = time_steps(torch, fn, 1, steps, warmup, reps, probes, filler=1)
    # outputs of each launch pattern for the oracle check (layer 0)
    for name, fn in (("grouped", sweep_grouped), ("device_list", sweep_list)):
        for li in range(36):
            for y_ in ys[li]:
                y_.fill_(float("nan"))
        fn(0)
        torch.cuda.synchronize()
        out[f"layer0_y_{name}"] = [ys[0][pi].cpu().numpy() for pi in range(7)]
    out["layer0_x"] = [x_host[0][which_x[pi]] for pi in range(7)]
    del mats
    torch.cuda.empty_cache()
    # the same 144 launches as plain streaming reads of each launch's bytes, over a 2.04 GB buffer
    sizes = []
    for _ in range(36):
        for grp in groups:
            sizes.append(sum(algorithmic_bytes("nvfp4", layer[pi][1], layer[pi][2]) for pi in grp))
    offs = np.concatenate([[0], np.cumsum([-(-b // 256) * 256 for b in sizes])]).astype(np.int64)
    buf = torch.empty(int(offs[-1]), dtype=torch.uint8, device="cuda")
    buf.random_(0, 256)
    base = buf.data_ptr()

    def probe_sweep(_):
        for j, b in enumerate(sizes):
            probes.read(base + int(offs[j]), b)

    out["read_probe"] = time_steps(torch, probe_sweep, 1, steps, warmup, reps, probes, filler=1)

    def one_read(_):
        probes.read(base, total_bytes)

    out["read_probe_one_launch"] = time_steps(torch, one_read, 1, steps, warmup, reps, probes, filler=1)
    del buf
    return out


def bench_packers(fp4, torch, synth, reps: int):
    """Throughput of the device packers on the 4096 x 4096 Dual workload's fp32 weights (load time, not the
    product): each packer call timed over a few launches, in weights per second and fp32 input GB/s."""
    n, k = synth.WORKLOADS[1]["shapes"][0]
    w = torch.from_numpy(synth.workload_weights(1, 0)).cuda()
    out = {}
    for fmt in ("rocmfp4_dual", "rocmfp4_fast", "nvfp4", "q4_0"):
        if fmt == "nvfp4":
            wq = torch.empty(n * k // 2, dtype=torch.uint8, device="cuda")
            ws = torch.empty(n * k // 16, dtype=torch.uint8, device="cuda")
            gb = torch.empty(1, dtype=torch.float32, device="cuda")

            def launch(_):
                fp4.fp4_quantize_nvfp4(n, k, w, wq, ws, gb)
        else:
            blocks = torch.empty(n * (k // 32) * BLOCK_BYTES[fmt], dtype=torch.uint8, device="cuda")
            if fmt == "q4_0":
                def launch(_):
                    fp4.fp4_quantize_q4_0(n, k, w, blocks)
            else:
                def launch(_, fmt=fmt):
                    fp4.fp4_quantize_rocmfp4(fmt, n, k, w, None, blocks)
        t = time_steps(torch, launch, 5, 5, 2, reps, None, filler=1)
        out[fmt] = {"ms": round(t["median_s"] * 1e3, 4), "Gweights/s": round(n * k / t["median_s"] / 1e9, 2),
                    "fp32_input_GB/s": round(4 * n * k / t["median_s"] / 1e9, 1), "timing": timing_fields(t)}
    return out


# ----------------------------------------------------------------------------------------------
# CPU baseline and the parity gate (the only part of this file that uses the oracle)

def _oracle_pack_rows(fmt: str, w_full: np.ndarray, rows: np.ndarray):
    """Oracle-packed canonical bytes of `rows` of w_full (NVFP4's global scale comes from the whole matrix)."""
    from oracle import pack
    if fmt == "nvfp4":
        return pack.pack_nvfp4_rows(w_full[rows], pack.nvfp4_global_scale(w_full))
    return pack.pack(fmt, np.ascontiguousarray(w_full[rows]))


def oracle_sample(fmt: str, w_full: np.ndarray, rows: np.ndarray, x_bits: np.ndarray, y_gpu: np.ndarray,
                  threads: int, budget_s: float, time_it: bool = True):
    """Time the oracle's exact dequant + FP64 product on `rows` of the matrix (on `threads` host threads, a
    slab of rows each) and compare y_gpu[:, rows] with it. Packing is input preparation, not timed."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from oracle import ref
    packed = _oracle_pack_rows(fmt, w_full, rows)
    parts = [p for p in np.array_split(np.arange(len(rows)), threads) if len(p)]
    chunks = [ref.rows(fmt, packed, p) for p in parts]

    def one(chunk):
        return ref.matmul(x_bits, ref.dequant(fmt, chunk))

    times = []
    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=len(chunks)) as ex:
        t_end = time.perf_counter() + budget_s
        while True:
            t0 = time.perf_counter()
            y_ref = np.concatenate(list(ex.map(one, chunks)), axis=1)
            times.append(time.perf_counter() - t0)
            if not time_it or (time.perf_counter() >= t_end and len(times) >= 3):
                break
    w64 = ref.dequant(fmt, packed)
    ok, worst = ref.check(y_gpu[:, rows], y_ref, ref.bound(x_bits, w64))
    n, k = len(rows), w_full.shape[1]
    med = float(np.median(times))
    m = x_bits.shape[0]
    return dict(parity=bool(ok), worst_error_ratio=float(f"{float(worst):.4g}"), rows=int(n), K=int(k), M=int(m),
                ms=round(med * 1e3, 3), runs=len(times),
                gbs=algorithmic_bytes(fmt, n, k) / med / 1e9, gflops=2.0 * m * n * k / med / 1e9)


def sample_rows(n: int, count: int) -> np.ndarray:
    return np.unique(np.linspace(0, n - 1, min(n, count)).astype(np.int64))


# ----------------------------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000, help="timed launches of the headline GEMV per repetition")
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--reps", type=int, default=5, help="timed repetitions per workload (median and spread)")
    ap.add_argument("--only", default="", help=f"comma-separated sections to run, of {','.join(SECTIONS)}")
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOADS),
                    help="the one-matrix GEMV workload of the headline figure")
    # The GEMM's clocks take tens of milliseconds of matrix-core load to settle (from ~245 to ~207 us per
    # launch on MI355X); the default warm-up covers that, so the timed launches measure steady state.
    ap.add_argument("--gemm-steps", type=int, default=100)
    ap.add_argument("--gemm-warmup", type=int, default=200)
    ap.add_argument("--spec-steps", type=int, default=400)
    ap.add_argument("--sweep-steps", type=int, default=10)
    ap.add_argument("--sweep-warmup", type=int, default=10)
    ap.add_argument("--cpu-budget", type=float, default=1.5, help="seconds of oracle timing per sampled workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline and the parity gate")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 256 MiB device copy (scale factor for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "the library and this benchmark run on one GPU; sharding across GPUs is "
                                   "described, not implemented (run with --gpus 1)", "n_gpus": args.gpus}))
        sys.exit(2)
    only = set(s for s in args.only.split(",") if s) or set(SECTIONS)
    unknown = only - set(SECTIONS)
    if unknown:
        ap.error(f"unknown sections {sorted(unknown)}")

    import torch
    import block_scaled_fp4_w4a16_amd as fp4
    import synth

    torch.cuda.set_device(0)
    torch.cuda.synchronize()
    if args.copy_calibration:
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 256)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"bytes_read": n, "bytes_written": n, "reps": 5}}), flush=True)
        return

    probes = Probes(torch)
    reps = max(1, args.reps)

    def log(msg):
        print(f"# {msg}", file=sys.stderr, flush=True)

    gemv_rows = {}          # name -> bench_gemv result
    read_probe = {}
    if "headline" in only:
        t0 = time.time()
        r = bench_gemv(fp4, torch, synth, args.workload, args.steps, args.warmup, reps, probes)
        gemv_rows[args.workload] = r
        log(f"gemv {args.workload}: {r['t']['median_s'] * 1e6:.3f} us/launch median "
            f"[{r['t']['min_s'] * 1e6:.3f}, {r['t']['max_s'] * 1e6:.3f}], "
            f"{r['bytes'] / r['t']['median_s'] / 1e9:.1f} GB/s "
            f"({r['copies']} cold copies, {time.time() - t0:.1f}s)")
    if "nvfp4_2048" in only:
        r = bench_gemv(fp4, torch, synth, "nvfp4_2048x2048_m1", args.steps, args.warmup, reps, probes)
        gemv_rows[r["name"]] = r
        log(f"gemv nvfp4_2048x2048_m1: {r['t']['median_s'] * 1e6:.3f} us/launch median")
    if "spec" in only:
        t0 = time.time()
        for fmt in SPEC_FMTS:
            for shape, _ in SPEC_SHAPES:
                for m in SPEC_MS:
                    name = f"{fmt}_{shape}_m{m}"
                    r = bench_gemv(fp4, torch, synth, name, args.spec_steps, args.spec_steps // 4, reps, probes)
                    gemv_rows[name] = r
        log(f"speculative-verify shapes: {len(SPEC_FMTS) * len(SPEC_SHAPES) * len(SPEC_MS)} workloads "
            f"({time.time() - t0:.1f}s)")
    if "read_probe" in only:
        t0 = time.time()
        sizes = sorted({algorithmic_bytes("nvfp4", 2048, 2048), algorithmic_bytes("rocmfp4_dual", 4096, 4096),
                        algorithmic_bytes("nvfp4", 9728, 2560), algorithmic_bytes("rocmfp4_fast", 9728, 2560)})
        for b in sizes:
            read_probe[b] = bench_read_probe(torch, probes, b, args.steps, args.warmup, reps)
        log(f"read probe: {len(sizes)} sizes ({time.time() - t0:.1f}s)")

    gemv_large = {}
    if "gemv_large" in only:
        t0 = time.time()
        for (n, k) in LARGE_SHAPES:
            for fmt in LARGE_FMTS:
                r = bench_gemv_large(fp4, torch, synth, fmt, n, k, 200, 100, reps, probes)
                gemv_large[r["name"]] = r
        log(f"large-matrix GEMV: " + ", ".join(f"{nm} {r['t']['median_s'] * 1e6:.2f} us" for nm, r in gemv_large.items())
            + f" ({time.time() - t0:.1f}s)")

    gemm, gemm_dense = {}, None
    if "gemm" in only:
        for fmt in ("rocmfp4_fast", "nvfp4"):
            t0 = time.time()
            gemm[fmt] = bench_gemm(fp4, torch, synth, fmt, 2048, args.gemm_steps, args.gemm_warmup, reps, probes)
            log(f"gemm {fmt} M=2048: {gemm[fmt]['t']['median_s'] * 1e6:.1f} us/launch median, "
                f"{gemm[fmt]['tflops']:.1f} TFLOP/s "
                f"({time.time() - t0:.1f}s)")
        t0 = time.time()
        gemm_dense = bench_dense_bf16_gemm(torch, 2048, 14336, 4096, args.gemm_steps, args.gemm_warmup, reps)
        log(f"dense bf16 linear M=2048: {gemm_dense['median_s'] * 1e6:.1f} us/launch median ({time.time() - t0:.1f}s)")
    gemm_small, gemm_small_n = {}, {}
    if "gemm_small" in only:
        t0 = time.time()
        pw = gemm["rocmfp4_fast"]["pw"] if "rocmfp4_fast" in gemm else None
        for m in (128, 256, 512):
            r = bench_gemm(fp4, torch, synth, "rocmfp4_fast", m, 200, 100, reps, probes, pw=pw)
            pw = r["pw"]
            gemm_small[m] = r
        # small N and long K (the 2560 x 9728 down projection of the verify workload): K parts in a workspace
        r = bench_gemm(fp4, torch, synth, "rocmfp4_fast", 128, 200, 100, reps, probes, cfg=3, mat=1)
        gemm_small_n = {128: r}
        log(f"gemm FAST small M ({time.time() - t0:.1f}s)")
    for r in gemm.values():
        r.pop("pw", None)
    for r in list(gemm_small.values()) + list(gemm_small_n.values()):
        r.pop("pw", None)

    sw = None
    if "sweep" in only:
        t0 = time.time()
        sw = bench_decode_sweep(fp4, torch, synth, args.sweep_steps, args.sweep_warmup, reps, probes)
        log(f"decode sweep: grouped {sw['grouped']['median_s'] * 1e6:.1f} us, single "
            f"{sw['single']['median_s'] * 1e6:.1f} us, device list {sw['device_list']['median_s'] * 1e6:.1f} us, "
            f"read probe {sw['read_probe']['median_s'] * 1e6:.1f} us "
            f"({time.time() - t0:.1f}s)")

    packers = None
    if "packers" in only:
        t0 = time.time()
        packers = bench_packers(fp4, torch, synth, reps)
        log(f"packers 4096x4096: " + ", ".join(f"{f} {v['ms']} ms" for f, v in packers.items())
            + f" ({time.time() - t0:.1f}s)")

    # ------------------------------------------------------------------ oracle: CPU baseline + parity gate
    cpu = {}
    threads = host_threads()
    if not args.no_cpu:
        t0 = time.time()
        budget = args.cpu_budget
        for name, r in gemv_rows.items():
            timed = (name in (HEADLINE, "nvfp4_2048x2048_m1") or r["m"] == 9)
            cpu[name] = oracle_sample(r["fmt"], r["w_np"], sample_rows(r["n"], 512), r["x_bits"], r["y"], threads,
                                      budget, time_it=timed)
        if gemm or gemm_small:
            w_pref = synth.workload_weights(4, 0)
            for fmt, r in gemm.items():
                cpu[f"{fmt}_prefill_m2048"] = oracle_sample(fmt, w_pref, sample_rows(r["n"], 64), r["x_bits"], r["y"],
                                                            threads, budget)
            for m, r in gemm_small.items():
                cpu[f"rocmfp4_fast_prefill_m{m}"] = oracle_sample("rocmfp4_fast", w_pref, sample_rows(r["n"], 64),
                                                                  r["x_bits"], r["y"], threads, budget, time_it=False)
            del w_pref
            if gemm_small_n:
                w_down = synth.workload_weights(3, 1)
                for m, r in gemm_small_n.items():
                    cpu[f"rocmfp4_fast_down_m{m}"] = oracle_sample("rocmfp4_fast", w_down, sample_rows(r["n"], 64),
                                                                   r["x_bits"], r["y"], threads, budget, time_it=False)
                del w_down
        for name, r in gemv_large.items():
            w = synth.device_weights(r["n"], r["k"], cfg=LARGE_CFG, mat=r["mat"]).cpu().numpy()
            cpu[name] = oracle_sample(r["fmt"], w, sample_rows(r["n"], 64), r["x_bits"], r["y"], threads, budget,
                                      time_it=False)
            del w
        if sw is not None:
            layer = synth.DECODE_4B_LAYER
            for mode in ("grouped", "device_list"):
                res = []
                for pi, (_, n, k) in enumerate(layer):
                    w = synth.device_weights(n, k, cfg=2, mat=pi).cpu().numpy()
                    res.append(oracle_sample("nvfp4", w, sample_rows(n, 256), sw["layer0_x"][pi],
                                             sw[f"layer0_y_{mode}"][pi], threads, budget / 7,
                                             time_it=(mode == "grouped")))
                cpu[f"decode_sweep_layer0_{mode}"] = dict(
                    parity=all(x["parity"] for x in res), worst_error_ratio=max(x["worst_error_ratio"] for x in res),
                    rows=sum(x["rows"] for x in res), ms=round(sum(x["ms"] for x in res), 3),
                    gbs=sum(algorithmic_bytes("nvfp4", x["rows"], x["K"]) for x in res)
                    / (sum(x["ms"] for x in res) / 1e3) / 1e9)
        log(f"oracle samples: {len(cpu)} ({time.time() - t0:.1f}s), parity "
            f"{'ok' if all(c['parity'] for c in cpu.values()) else 'FAILED: ' + str([k for k, c in cpu.items() if not c['parity']])}")

    def parity_of(key):
        c = cpu.get(key)
        return None if c is None else c["parity"]

    def gated(value, key):
        """No throughput for a workload whose oracle check failed."""
        return None if parity_of(key) is False else value

    # ------------------------------------------------------------------ the JSON line
    line = {"metric": "W4A16 GEMV weight GB/s & % HBM peak (M=1); GEMM TFLOP/s & % MFMA (M=2048)"}
    head = gemv_rows.get(args.workload)
    if head is not None:
        gbs = head["bytes"] / head["t"]["median_s"] / 1e9
        line.update({
            "value": gated(round(gbs, 2), args.workload),
            "unit": "GB/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": head["t"]["median_s"] * 1e3,
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic (seeded Student-t weights packed on the GPU by the library's packers; bf16 N(0,1) x)",
            "config": {"workload": args.workload, "fmt": head["fmt"], "M": head["m"], "N": head["n"],
                       "K": head["k"], "bytes_per_launch": head["bytes"], "cold_copies": head["copies"]},
            "roofline": hbm_roofline(head["bytes"], head["t"], traffic_from_profiles("gemv.hip", args.workload)),
            "timing": timing_fields(head["t"]),
            "parity": parity_of(args.workload),
        })
        if head["bytes"] in read_probe:
            rp = read_probe[head["bytes"]]
            line["roofline"]["vs_read_probe"] = round(rp["median_s"] / head["t"]["median_s"], 4)
    if not args.no_cpu and args.workload in cpu:
        c = cpu[args.workload]
        line["cpu_baseline"] = {
            "value": c["gbs"], "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{c['rows']} of {head['n']} rows x K={c['K']} ({head['fmt']}, M={c['M']}): exact dequant + "
                      f"FP64 product, one row slab per thread on {threads} threads, median of {c['runs']} runs "
                      f"({c['ms']} ms)",
            "cpu_model": cpu_model(),
            "per_workload": {k_: {f: v_[f] for f in ("ms", "gbs", "gflops", "rows", "M", "K", "runs", "parity",
                                                     "worst_error_ratio") if f in v_}
                             for k_, v_ in cpu.items()},
        }
    workloads = {}
    for name, r in gemv_rows.items():
        if name == args.workload:
            continue
        gbs = r["bytes"] / r["t"]["median_s"] / 1e9
        entry = {"fmt": r["fmt"], "N": r["n"], "K": r["k"], "M": r["m"], "bytes_per_launch": r["bytes"],
                 "GB/s": gated(round(gbs, 2), name), "roofline": hbm_roofline(r["bytes"], r["t"]),
                 "timing": timing_fields(r["t"]), "parity": parity_of(name), "cold_copies": r["copies"]}
        if r["bytes"] in read_probe:
            entry["roofline"]["vs_read_probe"] = round(read_probe[r["bytes"]]["median_s"] / r["t"]["median_s"], 4)
        # counter traffic where profiles/ holds it for the current kernel source (else null)
        entry["roofline"]["traffic"] = traffic_from_profiles("gemv.hip", name)
        workloads[name] = entry
    if workloads:
        line["gemv_workloads"] = workloads
    if gemv_large:
        line["gemv_large"] = {
            "what": "context: the M = 1 GEMV on large matrices (launch cost and latency amortised), N(0, 0.02) weights "
                    "packed on the GPU, a plain streaming read of the same bytes beside each",
            "results": {}}
        for name, r in gemv_large.items():
            gbs = r["bytes"] / r["t"]["median_s"] / 1e9
            rl = hbm_roofline(r["bytes"], r["t"])
            rl["vs_read_probe"] = round(r["t_read"]["median_s"] / r["t"]["median_s"], 4)
            line["gemv_large"]["results"][name] = {
                "fmt": r["fmt"], "N": r["n"], "K": r["k"], "M": 1, "bytes_per_launch": r["bytes"],
                "GB/s": gated(round(gbs, 2), name), "roofline": rl, "timing": timing_fields(r["t"]),
                "read_probe_GB/s": round(r["bytes"] / r["t_read"]["median_s"] / 1e9, 2),
                "parity": parity_of(name), "cold_copies": r["copies"]}
    if read_probe:
        line["read_probe"] = {
            "what": "plain streaming read of the same bytes per launch (16-byte nontemporal loads), cold copies",
            "results": {str(b): {"GB/s": round(b / t["median_s"] / 1e9, 2),
                                 "frac": round(b / t["median_s"] / 1e9 / HBM_PEAK_GBS, 4), **timing_fields(t)}
                        for b, t in read_probe.items()}}
    if gemm:
        line["gemm"] = {}
        for fmt, r in gemm.items():
            key = f"{fmt}_prefill_m2048"
            line["gemm"][f"{fmt}_prefill_m2048_k4096_n14336"] = {
                "TFLOP/s": gated(round(r["tflops"], 2), key),
                "roofline": {"bound": "mfma", "achieved": round(r["tflops"], 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(r["tflops"] / BF16_MFMA_PEAK_TFLOPS, 4),
                             "traffic": traffic_from_profiles("gemm.hip", f"{fmt}_prefill_m2048")},
                "timing": timing_fields(r["t"]), "parity": parity_of(key)}
    if gemm_dense is not None:
        tf = 2.0 * 2048 * 14336 * 4096 / gemm_dense["median_s"] / 1e12
        line["gemm_dense_bf16_context"] = {
            "what": "y = x W^T of the prefill shape on plain bf16 weights stored N x K (torch.nn.functional.linear, "
                    "ROCm BLAS library, no dequantization, bf16 output): context for the W4A16 GEMM, not a product "
                    "of this library",
            "TFLOP/s": round(tf, 2), "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4), "timing": timing_fields(gemm_dense)}
    if gemm_small:
        line["gemm_small_m"] = {
            f"rocmfp4_fast_m{m}_k4096_n14336": {
                "TFLOP/s": gated(round(r["tflops"], 2), f"rocmfp4_fast_prefill_m{m}"),
                "frac": round(r["tflops"] / BF16_MFMA_PEAK_TFLOPS, 4), "timing": timing_fields(r["t"]),
                "parity": parity_of(f"rocmfp4_fast_prefill_m{m}")} for m, r in gemm_small.items()}
    if gemm_small_n:
        line["gemm_small_n"] = {
            f"rocmfp4_fast_down_m{m}_k{r['k']}_n{r['n']}": {
                "TFLOP/s": gated(round(r["tflops"], 2), f"rocmfp4_fast_down_m{m}"),
                "frac": round(r["tflops"] / BF16_MFMA_PEAK_TFLOPS, 4), "timing": timing_fields(r["t"]),
                "k_parts": r["ws_bytes"] // (4 * m * r["n"]) if r["ws_bytes"] else 1,
                "parity": parity_of(f"rocmfp4_fast_down_m{m}")} for m, r in gemm_small_n.items()}
    if sw:
        g = sw["grouped"]
        gbs = sw["bytes"] / g["median_s"] / 1e9
        line["decode_sweep"] = {
            "workload": "nvfp4_4b_decode_sweep_m1 (36 layers x q,k,v,o,gate,up,down)",
            "GB/s": gated(round(gbs, 2), "decode_sweep_layer0_grouped"), "bytes_per_sweep": sw["bytes"],
            "launches_per_sweep": 144, "roofline": hbm_roofline(sw["bytes"], g), "timing": timing_fields(g),
            "parity": parity_of("decode_sweep_layer0_grouped"),
            "device_list": {
                "what": "the 252 products in launches of up to 32 matrices each (independent products; a decoder's "
                        "layers depend on each other and could not share launches)",
                "GB/s": gated(round(sw["bytes"] / sw["device_list"]["median_s"] / 1e9, 2),
                              "decode_sweep_layer0_device_list"),
                "launches_per_sweep": sw["list_launches"], "roofline": hbm_roofline(sw["bytes"], sw["device_list"]),
                "timing": timing_fields(sw["device_list"]), "parity": parity_of("decode_sweep_layer0_device_list")},
            "one_launch_per_matrix": {"GB/s": round(sw["bytes"] / sw["single"]["median_s"] / 1e9, 2),
                                      "launches_per_sweep": 252, "timing": timing_fields(sw["single"])},
            "read_probe_144_launches": {"GB/s": round(sw["bytes"] / sw["read_probe"]["median_s"] / 1e9, 2),
                                        "timing": timing_fields(sw["read_probe"])},
            "read_probe_one_launch": {"GB/s": round(sw["bytes"] / sw["read_probe_one_launch"]["median_s"] / 1e9, 2),
                                      "timing": timing_fields(sw["read_probe_one_launch"])},
        }
        line["decode_sweep"]["roofline"]["vs_read_probe"] = round(sw["read_probe"]["median_s"] / g["median_s"], 4)
    if packers:
        line["packers"] = {"workload": "device packers on the 4096 x 4096 fp32 weights (load time; ROCmFP4 with the "
                                       "pruned exhaustive-equivalent scale search)", "results": packers}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
