"""The GEMM entry point that allocates nothing (w4a16_gemm_noalloc: its K-part planes live in a static
device array) against the workspace entry point w4a16_gemm_ws given the workspace the library asks for:
the same launch, so the same bits, on two calls in a row, the second with a smaller input (the array keeps
the first call's contents, which the second must not depend on)."""
import numpy as np
import pytest
import torch

import synth
from tests import gpu_cases as gc

fp4 = pytest.importorskip("block_scaled_fp4_w4a16_amd")

pytestmark = pytest.mark.gpu


def test_gemm_noalloc_matches_workspace_entry():
    for fmt in ("nvfp4", "rocmfp4_dual"):
        for (m, n, k) in [(128, 2560, 9728), (65, 1000, 1152)]:   # the second call is smaller
            print("CASE gemm-noalloc", fmt, m, n, k, flush=True)
            need = fp4.w4a16_gemm_workspace_bytes(fmt, m, n, k)
            assert 0 < need <= (16 << 20)       # K parts in the static array, within its size
            w, packed = gc.make_case(fmt, n, k, cfg=78, mat=m)
            del w
            pw = gc.upload(fmt, n, k, packed)
            x_bits = synth.activations(m, k, cfg=78, mat=m)
            x = gc.x_tensor(x_bits)
            ws = torch.empty(need, dtype=torch.uint8, device="cuda")
            y_ws = torch.full((m, n), float("nan"), device="cuda")
            fp4.w4a16_gemm(fmt, m, n, k, pw.q, pw.s, pw.global_scale, x, y_ws, workspace=ws)
            y_na = torch.full((m, n), float("nan"), device="cuda")
            fp4.w4a16_gemm_noalloc(fmt, m, n, k, pw.q, pw.s, pw.global_scale, x, y_na)
            torch.cuda.synchronize()
            assert torch.equal(y_na, y_ws), (fmt, m, n, k)
            cols = np.unique(np.concatenate([[0, n - 1], np.linspace(0, n - 1, 16).astype(int)]))
            gc.check_product(fmt, packed, x_bits, y_na, cols=cols, label=f"gemm-noalloc {fmt} M={m} {n}x{k}")
