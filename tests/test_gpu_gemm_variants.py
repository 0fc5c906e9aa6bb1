"""GPU: the shared-decode GEMM kernel (decode each weight tile once into a bf16 LDS tile that 8 waves read as
MFMA B operands), selected with FP4_GEMM_LDS=1, against the default GEMM kernel and the oracle. The same
products are summed in the same order, so the outputs must be bitwise equal."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import synth
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu

fp4 = pytest.importorskip("block_scaled_fp4_w4a16_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (M, N, K): one tile, a ragged grid, several bands with a ragged last band, ragged N
CASES = [(256, 256, 128), (300, 700, 512), (1200, 4352, 2048), (2048, 2304, 1024)]


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_shared_decode_gemm_matches_default_kernel_bitwise(tmp_path):
    want = {}
    for fmt in gc.FMTS:
        for (m, n, k) in CASES:
            name = f"{fmt}__{m}__{n}__{k}"
            print("CASE default", name, flush=True)
            w, packed = gc.make_case(fmt, n, k, cfg=98, mat=m)
            pw = gc.upload(fmt, n, k, packed)
            xb = synth.activations(m, k, cfg=98, mat=m)
            y = torch.empty(m, n, dtype=torch.float32, device="cuda")
            fp4.w4a16_gemm(fmt, m, n, k, pw.q, pw.s, pw.global_scale, gc.x_tensor(xb), y)
            torch.cuda.synchronize()
            cols = np.unique(np.linspace(0, n - 1, 24).astype(int))
            gc.check_product(fmt, packed, xb, y, cols=cols, label=f"default {name}")
            want[name] = y.cpu().numpy()
            for key, arr in (("q", pw.q), ("s", pw.s)):
                np.save(tmp_path / f"{name}.{key}.npy", arr.cpu().numpy())
            np.save(tmp_path / f"{name}.g.npy", np.float32(pw.global_scale))
            np.save(tmp_path / f"{name}.x.npy", xb)
    env = dict(os.environ, FP4_GEMM_LDS="1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "gemm_variant_child.py"), str(tmp_path)],
                       env=env, capture_output=True, text=True, timeout=300)
    print(r.stdout[-2000:], r.stderr[-2000:])
    assert r.returncode == 0
    for name, y0 in want.items():
        y1 = np.load(tmp_path / f"{name}.y_variant.npy")
        assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32)), name
