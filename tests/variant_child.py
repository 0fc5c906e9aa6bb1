"""Child process of the GPU tests that force a kernel variant. The library reads its tuning overrides
(FP4_GEMM_SHORT, FP4_GEMM_SPLIT, FP4_GEMM_BAND_ROWS, FP4_GEMV_RING, FP4_QUANT_EXHAUSTIVE, ...) once per process, so
a forced variant needs a process of its own: this one runs the products the parent saved in `folder`
(one .npz per case: entry, fmt, m, n, k, planes q and s, global scale g, x; or, for the ROCmFP4 packer,
weights w and optionally importance imp) and saves each output as <case>.y.npy beside it."""
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import block_scaled_fp4_w4a16_amd as fp4  # noqa: E402


def main(folder: str):
    for f in sorted(os.listdir(folder)):
        if not f.endswith(".npz"):
            continue
        d = np.load(os.path.join(folder, f))
        entry, fmt = str(d["entry"]), str(d["fmt"])
        m, n, k = int(d["m"]), int(d["n"]), int(d["k"])
        print("CASE", f, entry, fmt, m, n, k, flush=True)
        if entry == "quant":  # the ROCmFP4 device packer: fp32 w[n][k] (and importance) -> canonical blocks
            w = torch.from_numpy(d["w"]).cuda()
            imp = torch.from_numpy(d["imp"]).cuda() if "imp" in d.files else None
            blocks = torch.empty(n * (k // 32) * fp4.BLOCK_BYTES[fmt], dtype=torch.uint8, device="cuda")
            fp4.fp4_quantize_rocmfp4(fmt, n, k, w, imp, blocks)
            torch.cuda.synchronize()
            np.save(os.path.join(folder, f[:-4] + ".y.npy"), blocks.cpu().numpy())
            continue
        q = torch.from_numpy(d["q"]).cuda()
        s = torch.from_numpy(d["s"]).cuda()
        x = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).cuda()
        y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
        getattr(fp4, {"gemm": "w4a16_gemm", "gemv": "w4a16_gemv"}[entry])(fmt, m, n, k, q, s, float(d["g"]), x, y)
        torch.cuda.synchronize()
        np.save(os.path.join(folder, f[:-4] + ".y.npy"), y.cpu().numpy())
    print("child done", flush=True)


if __name__ == "__main__":
    main(sys.argv[1])
