"""GPU: kernel variants that a tuning override selects, each in a child process (the library reads its
overrides once per process), against the default kernels:
  * the exhaustive ROCmFP4 packer (every candidate scored), FP4_QUANT_EXHAUSTIVE=1, against the default
    pruned search: byte-equal blocks, on groups that exercise both pruned directions, ties, zero and
    negative importance (negative importance switches pruning off) and extreme magnitudes."""
import numpy as np
import pytest
import torch

import synth
from oracle import pack
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu

fp4 = pytest.importorskip("block_scaled_fp4_w4a16_amd")


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_pruned_packer_matches_exhaustive_kernel(tmp_path):
    rng = np.random.default_rng(5)
    cases = {}
    for fmt in ("rocmfp4_dual", "rocmfp4_fast"):
        for name, n, k in (("t", 64, 512), ("outl", 48, 1024), ("edge", 16, 256)):
            if name == "edge":
                w = np.zeros((n, k), np.float32)
                s = np.float32(0.8125)
                w[0] = (rng.choice([0, 0.5, 1.5, 2.5, 3.5, 5, 7, 9, 10, 30], size=k) * s).astype(np.float32)
                w[1] = 1e-7 * rng.standard_normal(k).astype(np.float32)
                w[2] = 3000.0 * rng.standard_normal(k).astype(np.float32)
                w[3:] = synth.weights(n - 3, k, dist="t", nu=3.0, cfg=130, mat=1)
            else:
                w = synth.weights(n, k, dist="t", nu=4.0, outlier_frac=0.0 if name == "t" else 0.01, cfg=131,
                                  mat=n)
            for imp_kind in ("none", "pos", "neg"):
                case = f"{fmt}_{name}_{imp_kind}"
                print("CASE", case, flush=True)
                imp = None
                if imp_kind != "none":
                    imp = np.abs(rng.standard_normal((n, k))).astype(np.float32)
                    imp[rng.random((n, k)) < 0.2] = 0.0
                    if imp_kind == "neg":
                        imp[rng.random((n, k)) < 0.05] *= -1.0
                blocks = torch.empty(n * (k // 32) * fp4.BLOCK_BYTES[fmt], dtype=torch.uint8, device="cuda")
                fp4.fp4_quantize_rocmfp4(fmt, n, k, torch.from_numpy(w).cuda(),
                                         None if imp is None else torch.from_numpy(imp).cuda(), blocks)
                torch.cuda.synchronize()
                got = blocks.cpu().numpy()
                # the oracle's exhaustive search too (with a negative importance pruning is off, so the device
                # packer scores every candidate like the oracle)
                assert np.array_equal(got.reshape(n, k // 32, -1), pack.pack(fmt, w, importance=imp)[0]), case
                cases[case] = got
                arrays = dict(entry="quant", fmt=fmt, m=0, n=n, k=k, w=w)
                if imp is not None:
                    arrays["imp"] = imp
                np.savez(tmp_path / f"{case}.npz", **arrays)
    ys = gc.run_variant(tmp_path, {"FP4_QUANT_EXHAUSTIVE": "1"})
    for case, got in cases.items():
        assert np.array_equal(got, ys[case]), case
