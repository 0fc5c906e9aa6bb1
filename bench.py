"""Benchmark of the W4A16 hot path on one MI355X.

Default workload: ROCmFP4 Dual 4096 x 4096, M = 1 (decode GEMV), plus the prefill GEMM
(ROCmFP4 FAST, M = 2048, K = 4096, N = 14336) reported in the same JSON line.

A step is one GEMV launch over one packed matrix. Weights are drawn by `synth`, packed on the
GPU by the library's own packer (fp4_quantize_*), repacked to kernel layout and replicated into
enough distinct copies (>= 1 GiB) that every launch reads its matrix from HBM rather than from
the 256 MB last-level cache. Launches are recorded into HIP graphs on torch's current stream and
timed with HIP events on that stream between synchronisations; `value` is weight + scale bytes
per launch divided by the average launch time.

The `cpu_baseline` leg times the CPU oracle (exact dequantisation + FP64 product) on a bounded
row sample of the same workload, packed by the oracle itself.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
COLD_BYTES = 1 << 30            # 4x the 256 MB last-level cache
BLOCK_BYTES = {"rocmfp4_dual": 18, "rocmfp4_fast": 17, "q4_0": 18}

WORKLOADS = {
    # name: (synth cfg, matrix index, fmt, M)
    "rocmfp4_dual_4096x4096_m1": (1, 0, "rocmfp4_dual", 1),
    "nvfp4_2048x2048_m1": (0, 0, "nvfp4", 1),
    "nvfp4_gate_9728x2560_m1": (3, 0, "nvfp4", 1),
    "rocmfp4_dual_gate_9728x2560_m1": (3, 0, "rocmfp4_dual", 1),
    "rocmfp4_fast_gate_9728x2560_m1": (3, 0, "rocmfp4_fast", 1),
    "nvfp4_down_2560x9728_m1": (3, 1, "nvfp4", 1),
    "rocmfp4_dual_down_2560x9728_m1": (3, 1, "rocmfp4_dual", 1),
    "rocmfp4_fast_down_2560x9728_m1": (3, 1, "rocmfp4_fast", 1),
}
WORKLOADS["q4_0_4096x4096_m1"] = (1, 0, "q4_0", 1)          # the Dual matrix in stock Q4_0 (same bytes)
WORKLOADS["q4_0_gate_9728x2560_m1"] = (3, 0, "q4_0", 1)
WORKLOADS["q4_0_down_2560x9728_m1"] = (3, 1, "q4_0", 1)
for _m in (9, 16):
    for _f in ("nvfp4", "rocmfp4_dual", "rocmfp4_fast", "q4_0"):
        WORKLOADS[f"{_f}_gate_9728x2560_m{_m}"] = (3, 0, _f, _m)
        WORKLOADS[f"{_f}_down_2560x9728_m{_m}"] = (3, 1, _f, _m)


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


# ----------------------------------------------------------------------------------------------
def pack_on_gpu(fp4, torch, fmt: str, w_np: np.ndarray):
    """synth fp32 weights -> device packer -> kernel layout (all on the GPU, no oracle)."""
    w = torch.from_numpy(w_np).cuda()
    pw = fp4.PackedWeight.quantize(fmt, w)
    del w
    return pw


def replicate(torch, pw, copies: int):
    qs = [pw.q] + [pw.q.clone() for _ in range(copies - 1)]
    ss = [pw.s] + [pw.s.clone() for _ in range(copies - 1)]
    return qs, ss


def graph_of(torch, fn, launches):
    """Capture `launches` calls fn(i) into one HIP graph (the library launches on the capture stream)."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in launches:  # warm the code path outside capture once
            fn(i)
            break
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in launches:
            fn(i)
    torch.cuda.synchronize()
    return g


def time_launches(torch, fn, copies: int, steps: int, warmup: int):
    """Run `steps` launches (launch i uses copy i % copies) as graph replays; return seconds."""
    g_full = graph_of(torch, fn, range(copies))
    rem = steps % copies
    g_rem = graph_of(torch, fn, range(rem)) if rem else None
    for _ in range(max(1, warmup // copies)):
        g_full.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps // copies):
        g_full.replay()
    if g_rem is not None:
        g_rem.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3


def bench_gemv(fp4, torch, synth, name: str, steps: int, warmup: int):
    cfg, mat, fmt, m = WORKLOADS[name]
    n, k = synth.WORKLOADS[cfg]["shapes"][mat]
    w_np = synth.workload_weights(cfg, mat)
    pw = pack_on_gpu(fp4, torch, fmt, w_np)
    plane_bytes = pw.q.numel() + pw.s.numel()
    copies = max(2, -(-COLD_BYTES // plane_bytes))
    qs, ss = replicate(torch, pw, copies)
    x_bits = synth.workload_activations(cfg, mat, m)
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).cuda()
    ys = [torch.empty((m, n), dtype=torch.float32, device="cuda") for _ in range(min(copies, 8))]

    def launch(i):
        fp4.w4a16_gemv(fmt, m, n, k, qs[i], ss[i], pw.global_scale, x, ys[i % len(ys)])

    secs = time_launches(torch, launch, copies, steps, warmup)
    per_launch = secs / steps
    abytes = algorithmic_bytes(fmt, n, k)
    y0 = torch.empty((m, n), dtype=torch.float32, device="cuda")
    fp4.w4a16_gemv(fmt, m, n, k, qs[0], ss[0], pw.global_scale, x, y0)
    torch.cuda.synchronize()
    return dict(fmt=fmt, n=n, k=k, m=m, copies=copies, per_launch_s=per_launch, bytes=abytes,
                gbs=abytes / per_launch / 1e9, y0=y0.cpu().numpy(), x_bits=x_bits, w_np=w_np)


def bench_gemm(fp4, torch, synth, fmt: str, steps: int, warmup: int, m: int = 2048, pw=None):
    cfg, mat = 4, 0
    n, k = synth.WORKLOADS[cfg]["shapes"][mat]
    if pw is None:
        w_np = synth.workload_weights(cfg, mat)
        pw = pack_on_gpu(fp4, torch, fmt, w_np)
        del w_np
    x_bits = synth.workload_activations(cfg, mat, m)
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).cuda()
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")

    def launch(i):
        fp4.w4a16_gemm(fmt, m, n, k, pw.q, pw.s, pw.global_scale, x, y)

    copies = 1
    secs = time_launches(torch, launch, copies, steps, warmup)
    per = secs / steps
    flops = 2.0 * m * n * k
    return dict(fmt=fmt, m=m, n=n, k=k, per_launch_s=per, tflops=flops / per / 1e12, pw=pw)


def host_threads() -> int:
    """Host cores this process may use (the affinity mask), at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def bench_decode_sweep(fp4, torch, synth, steps: int, warmup: int):
    """The 4B-class decode sweep: 36 layers x {q, k, v, o, gate, up, down}, NVFP4, M = 1.

    Weights are N(0, 0.02) drawn on the GPU (synth.device_weights) and packed by the library's NVFP4
    packer; all 252 matrices (2.04 GB) stay resident, so each sweep streams them from HBM. A sweep is
    launched per layer the way a decoder consumes it: one grouped launch for q|k|v (same x), one for
    o, one grouped launch for gate|up (same x), one for down -- 144 launches. The same sweep with one
    launch per matrix (252 launches) is timed beside it. Both are recorded as HIP graphs.
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
        return torch.from_numpy(synth.activations(1, k, cfg=cfg, mat=mat).view(np.int16)).view(torch.bfloat16).cuda()

    xs = [dict(attn=xb(2560, 4 * li), o=xb(4096, 4 * li + 1), mlp=xb(2560, 4 * li + 2), down=xb(9728, 4 * li + 3))
          for li in range(36)]
    ys = [[torch.empty((1, n), dtype=torch.float32, device="cuda") for (_, n, _) in layer] for _ in range(36)]
    which_x = ("attn", "attn", "attn", "o", "mlp", "mlp", "down")

    def item(li, pi):
        pw = mats[li][pi]
        return (pw.q, pw.s, pw.global_scale, xs[li][which_x[pi]], ys[li][pi], pw.N, pw.K)

    def sweep_grouped(_):
        for li in range(36):
            fp4.w4a16_gemv_batched("nvfp4", 1, [item(li, 0), item(li, 1), item(li, 2)])
            fp4.w4a16_gemv_batched("nvfp4", 1, [item(li, 3)])
            fp4.w4a16_gemv_batched("nvfp4", 1, [item(li, 4), item(li, 5)])
            fp4.w4a16_gemv_batched("nvfp4", 1, [item(li, 6)])

    def sweep_single(_):
        for li in range(36):
            for pi in range(7):
                q, s_, g, x, y, n, k = item(li, pi)
                fp4.w4a16_gemv("nvfp4", 1, n, k, q, s_, g, x, y)

    out = dict(bytes=total_bytes)
    for name, fn in (("grouped", sweep_grouped), ("single", sweep_single)):
        secs = time_launches(torch, fn, 1, steps, warmup)
        out[name] = secs / steps
    return out


def cpu_baseline(fmt: str, w_np: np.ndarray, x_bits: np.ndarray, y_gpu: np.ndarray, budget_s: float = 12.0):
    """The CPU oracle on a row sample of the same matrix: oracle-packed, exact dequant + FP64 product."""
    from threadpoolctl import threadpool_limits

    from oracle import pack, ref
    threads = host_threads()
    rows = np.arange(0, w_np.shape[0], max(1, w_np.shape[0] // 512))[:512]
    sample_w = np.ascontiguousarray(w_np[rows])
    packed = pack.pack(fmt, sample_w)                       # input preparation, not timed
    n, k = sample_w.shape
    abytes = algorithmic_bytes(fmt, n, k)
    times = []
    with threadpool_limits(limits=threads):
        t_end = time.perf_counter() + budget_s
        while time.perf_counter() < t_end or len(times) < 3:
            t0 = time.perf_counter()
            w64 = ref.dequant(fmt, packed)
            y_ref = ref.matmul(x_bits, w64)
            times.append(time.perf_counter() - t0)
    med = float(np.median(times))
    b = ref.bound(x_bits, w64)
    ok, worst = ref.check(y_gpu[:, rows], y_ref, b)
    return dict(value=abytes / med / 1e9, unit="GB/s", cores=threads, kind="oracle",
                sample=f"{n} of {w_np.shape[0]} rows x K={k} ({fmt}, M={x_bits.shape[0]}), exact dequant "
                       f"(numpy, one thread) + FP64 product (BLAS, {threads} threads), median of "
                       f"{len(times)} runs",
                ms=med * 1e3, parity_on_sample=ok, worst_error_ratio=worst)


def copy_calibration(torch, mib: int = 256, reps: int = 5):
    """A plain device copy of known size, run so that rocprofv3 counters can be scaled to bytes."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 256)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": n, "bytes_written": n, "reps": reps}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=11400)
    ap.add_argument("--warmup", type=int, default=1140)
    ap.add_argument("--workload", default="rocmfp4_dual_4096x4096_m1", choices=sorted(WORKLOADS))
    # The GEMM's clocks take tens of milliseconds of matrix-core load to settle (from ~245 to ~207 us per
    # launch on MI355X); the default warmup covers that, so the timed launches measure steady state.
    ap.add_argument("--gemm-steps", type=int, default=200)
    ap.add_argument("--gemm-warmup", type=int, default=200)
    ap.add_argument("--no-gemm", action="store_true")
    ap.add_argument("--no-gemm-small", action="store_true", help="skip the M = 128, 256, 512 GEMM figures")
    ap.add_argument("--no-spec", action="store_true", help="skip the speculative-verify shapes (M = 1, 9, 16)")
    ap.add_argument("--spec-steps", type=int, default=2000)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--sweep-steps", type=int, default=50)
    ap.add_argument("--sweep-warmup", type=int, default=20)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 256 MiB device copy (scale factor for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "the library and this benchmark run on one GPU; sharding across GPUs is "
                                   "described, not implemented (run with --gpus 1)", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import block_scaled_fp4_w4a16_amd as fp4
    import synth

    torch.cuda.set_device(0)
    torch.cuda.synchronize()
    if args.copy_calibration:
        copy_calibration(torch)
        return
    t0 = time.time()
    gv = bench_gemv(fp4, torch, synth, args.workload, args.steps, args.warmup)
    print(f"# gemv {args.workload}: {gv['per_launch_s'] * 1e6:.3f} us/launch, {gv['gbs']:.1f} GB/s "
          f"({gv['copies']} cold copies, {time.time() - t0:.1f}s)", file=sys.stderr, flush=True)

    gm = None
    if not args.no_gemm:
        t1 = time.time()
        gm = bench_gemm(fp4, torch, synth, "rocmfp4_fast", args.gemm_steps, args.gemm_warmup)
        print(f"# gemm FAST M=2048: {gm['per_launch_s'] * 1e6:.1f} us/launch, {gm['tflops']:.1f} TFLOP/s "
              f"({time.time() - t1:.1f}s)", file=sys.stderr, flush=True)
        t1 = time.time()
        gm_nv = bench_gemm(fp4, torch, synth, "nvfp4", args.gemm_steps, args.gemm_warmup)
        print(f"# gemm NVFP4 M=2048: {gm_nv['per_launch_s'] * 1e6:.1f} us/launch, {gm_nv['tflops']:.1f} TFLOP/s "
              f"({time.time() - t1:.1f}s)", file=sys.stderr, flush=True)
        # the same FAST matrix at prefill-chunk sizes (small grids: two-way K split, 128/192-row tiles);
        # one weight copy, so the weights stay in the last-level cache between launches
        t1 = time.time()
        gm_small = {}
        for m_small in (() if args.no_gemm_small else (128, 256, 512)):
            r = bench_gemm(fp4, torch, synth, "rocmfp4_fast", 400, 200, m=m_small, pw=gm["pw"])
            gm_small[f"m{m_small}"] = {"us_per_launch": round(r["per_launch_s"] * 1e6, 2),
                                       "TFLOP/s": round(r["tflops"], 1)}
        print(f"# gemm FAST small M: {gm_small} ({time.time() - t1:.1f}s)", file=sys.stderr, flush=True)

    spec = None
    if not args.no_spec:
        # speculative verify / small batch: gate- and down-shaped matrices at M = 1, 9 (1 token + 8 drafts), 16
        t3 = time.time()
        spec = {}
        for fmt in ("nvfp4", "rocmfp4_dual"):
            for shape in ("gate_9728x2560", "down_2560x9728"):
                for m in (1, 9, 16):
                    name = f"{fmt}_{shape}_m{m}"
                    r = bench_gemv(fp4, torch, synth, name, args.spec_steps, args.spec_steps // 10)
                    spec[name] = {"us_per_launch": round(r["per_launch_s"] * 1e6, 3), "GB/s": round(r["gbs"], 1),
                                  "frac": round(r["gbs"] / HBM_PEAK_GBS, 4)}
        print(f"# speculative-verify shapes: {len(spec)} workloads ({time.time() - t3:.1f}s)", file=sys.stderr,
              flush=True)

    sw = None
    if not args.no_sweep:
        t2 = time.time()
        sw = bench_decode_sweep(fp4, torch, synth, args.sweep_steps, args.sweep_warmup)
        print(f"# decode sweep NVFP4 M=1 (252 matrices, {sw['bytes'] / 1e9:.3f} GB): grouped "
              f"{sw['grouped'] * 1e6:.1f} us ({sw['bytes'] / sw['grouped'] / 1e9:.1f} GB/s), one launch per matrix "
              f"{sw['single'] * 1e6:.1f} us ({sw['bytes'] / sw['single'] / 1e9:.1f} GB/s) ({time.time() - t2:.1f}s)",
              file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(gv["fmt"], gv["w_np"], gv["x_bits"], gv["y0"])
        print(f"# cpu oracle: {cpu['value']:.4f} GB/s on the sample, parity {cpu['parity_on_sample']}",
              file=sys.stderr, flush=True)

    line = {
        "metric": "W4A16 GEMV weight GB/s & % HBM peak (M=1); GEMM TFLOP/s & % MFMA (M=2048)",
        "value": round(gv["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": gv["per_launch_s"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Student-t weights packed on the GPU by the library's packer; bf16 N(0,1) x)",
        "config": {"workload": args.workload, "fmt": gv["fmt"], "M": gv["m"], "N": gv["n"], "K": gv["k"],
                   "bytes_per_launch": gv["bytes"], "cold_copies": gv["copies"]},
        "roofline": {"bound": "hbm", "achieved": round(gv["gbs"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gv["gbs"] / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profiles("gemv.hip", args.workload)},
        "cpu_baseline": cpu and {k_: cpu[k_] for k_ in ("value", "unit", "cores", "kind", "sample")},
    }
    if cpu:
        line["cpu_baseline"]["parity_on_sample"] = cpu["parity_on_sample"]
    if gm:
        line["gemm"] = {"workload": "rocmfp4_fast_prefill_m2048_k4096_n14336", "value": round(gm["tflops"], 2),
                        "unit": "TFLOP/s", "us_per_launch": round(gm["per_launch_s"] * 1e6, 2),
                        "steps": args.gemm_steps, "warmup": args.gemm_warmup,
                        "roofline": {"bound": "mfma", "achieved": round(gm["tflops"], 2),
                                     "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                     "frac": round(gm["tflops"] / BF16_MFMA_PEAK_TFLOPS, 4),
                                     "traffic": traffic_from_profiles("gemm.hip", "rocmfp4_fast_prefill_m2048")},
                        "nvfp4": {"workload": "nvfp4_prefill_m2048_k4096_n14336", "value": round(gm_nv["tflops"], 2),
                                  "us_per_launch": round(gm_nv["per_launch_s"] * 1e6, 2),
                                  "frac": round(gm_nv["tflops"] / BF16_MFMA_PEAK_TFLOPS, 4)},
                        "small_m": {"workload": "rocmfp4_fast k4096 n14336 at M = 128, 256, 512", **gm_small}}
    if spec:
        line["spec_verify"] = {"workload": "speculative verify, gate 9728x2560 and down 2560x9728, M = 1, 9, 16",
                               "unit": "GB/s of weight + scale bytes", "steps": args.spec_steps, "results": spec}
    if sw:
        gbs = sw["bytes"] / sw["grouped"] / 1e9
        line["decode_sweep"] = {
            "workload": "nvfp4_4b_decode_sweep_m1 (36 layers x q,k,v,o,gate,up,down)",
            "value": round(gbs, 2), "unit": "GB/s", "us_per_sweep": round(sw["grouped"] * 1e6, 2),
            "launches_per_sweep": 144, "bytes_per_sweep": sw["bytes"],
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4)},
            "one_launch_per_matrix": {"value": round(sw["bytes"] / sw["single"] / 1e9, 2),
                                      "us_per_sweep": round(sw["single"] * 1e6, 2), "launches_per_sweep": 252},
        }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
