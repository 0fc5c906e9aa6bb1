"""Helpers shared by the GPU parity tests: seeded inputs, oracle packing, upload, comparison."""
from __future__ import annotations

import numpy as np
import torch

import synth
from oracle import pack, ref

FMTS = ("nvfp4", "rocmfp4_dual", "rocmfp4_fast")   # every path, matrix-core GEMM and mid-M included
FMTS_ALL = FMTS + ("q4_0",)                          # the GEMV family and the dequantizer


def canonical_tensors(fmt, packed, device="cuda"):
    """Oracle-packed canonical bytes -> device tensors (src_q, src_s, g)."""
    if fmt == "nvfp4":
        wq, ws, g = packed
        return (torch.from_numpy(np.ascontiguousarray(wq)).reshape(-1).to(device),
                torch.from_numpy(np.ascontiguousarray(ws)).reshape(-1).to(device), float(g))
    blocks, g = packed
    return torch.from_numpy(np.ascontiguousarray(blocks)).reshape(-1).to(device), None, float(g)


def upload(fmt, n, k, packed):
    import block_scaled_fp4_w4a16_amd as fp4
    q, s, g = canonical_tensors(fmt, packed)
    pw = fp4.PackedWeight.from_canonical(fmt, n, k, q, s, g)
    torch.cuda.synchronize()
    return pw


def make_case(fmt, n, k, *, dist="t", nu=5.0, outlier_frac=0.0, cfg=50, mat=0):
    w = synth.weights(n, k, dist=dist, nu=nu, outlier_frac=outlier_frac, cfg=cfg, mat=mat)
    return w, pack.pack(fmt, w)


def x_tensor(x_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).cuda()


def check_product(fmt, packed, x_bits, y_gpu, cols=None, label=""):
    """Compare y_gpu [M, N] (or the columns `cols`) with the FP64 oracle; assert the tolerance."""
    sub = packed if cols is None else ref.rows(fmt, packed, cols)
    w64 = ref.dequant(fmt, sub)
    y_ref = ref.matmul(x_bits, w64)
    b = ref.bound(x_bits, w64)
    y = y_gpu.detach().cpu().numpy().astype(np.float64)
    if cols is not None:
        y = y[:, cols]
    ok, worst = ref.check(y, y_ref, b)
    assert ok, f"{label}: worst error / allowance = {worst}"
    return worst


def save_case(folder, name, entry, fmt, m, n, k, pw, x_bits):
    """Write one product's inputs for tests/variant_child.py."""
    import os
    np.savez(os.path.join(str(folder), name + ".npz"), entry=entry, fmt=fmt, m=m, n=n, k=k, q=pw.q.cpu().numpy(),
             s=pw.s.cpu().numpy(), g=np.float32(pw.global_scale), x=x_bits)


def run_variant(folder, env_overrides: dict) -> dict:
    """Run the saved cases in a child process with the given tuning overrides; returns {name: y}."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, **env_overrides)
    r = subprocess.run([sys.executable, os.path.join(root, "tests", "variant_child.py"), str(folder)], env=env,
                       capture_output=True, text=True, timeout=600)
    print(r.stdout[-3000:], r.stderr[-3000:], flush=True)
    assert r.returncode == 0, f"variant child failed with status {r.returncode}"
    out = {}
    for f in os.listdir(str(folder)):
        if f.endswith(".y.npy"):
            out[f[:-6]] = np.load(os.path.join(str(folder), f))
    return out
