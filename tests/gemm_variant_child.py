"""Child process of test_gpu_gemm_variants: runs w4a16_gemm on the inputs the parent saved, in this process's
kernel configuration (the library reads its tuning overrides once per process, so a forced kernel variant
needs a process of its own), and saves the outputs next to them."""
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import block_scaled_fp4_w4a16_amd as fp4  # noqa: E402


def main(folder: str):
    names = sorted(f[:-6] for f in os.listdir(folder) if f.endswith(".q.npy"))
    for name in names:
        fmt, m, n, k = name.split("__")
        m, n, k = int(m), int(n), int(k)
        print("CASE", name, flush=True)
        q = torch.from_numpy(np.load(os.path.join(folder, name + ".q.npy"))).cuda()
        s = torch.from_numpy(np.load(os.path.join(folder, name + ".s.npy"))).cuda()
        g = float(np.load(os.path.join(folder, name + ".g.npy")))
        xb = np.load(os.path.join(folder, name + ".x.npy"))
        x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda()
        y = torch.empty(m, n, dtype=torch.float32, device="cuda")
        fp4.w4a16_gemm(fmt, m, n, k, q, s, g, x, y)
        torch.cuda.synchronize()
        np.save(os.path.join(folder, name + ".y_variant.npy"), y.cpu().numpy())
    print("child done", flush=True)


if __name__ == "__main__":
    main(sys.argv[1])
