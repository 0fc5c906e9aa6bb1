"""Parity at the benchmark workloads' full sizes, through the same entry points and dispatch
the benchmark times. Weights are drawn by synth and packed by the CPU oracle; outputs are
checked against the FP64 oracle on every column (or, for the prefill GEMM, on sampled
columns over all rows)."""
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


def _run(fmt, cfg, mat, m, cols=None):
    wl = synth.WORKLOADS[cfg]
    n, k = wl["shapes"][mat]
    print("CASE workload", wl["name"], fmt, n, k, "M", m, flush=True)
    w = synth.workload_weights(cfg, mat)
    packed = pack.pack(fmt, w)
    pw = gc.upload(fmt, n, k, packed)
    x_bits = synth.workload_activations(cfg, mat, m)
    y = torch.full((m, n), float("nan"), device="cuda")
    fp4.w4a16_matmul(fmt, m, n, k, pw.q, pw.s, pw.global_scale, gc.x_tensor(x_bits), y)
    torch.cuda.synchronize()
    return gc.check_product(fmt, packed, x_bits, y, cols=cols, label=f"{wl['name']} {fmt} M={m}")


def test_nvfp4_2048x2048_m1():
    _run("nvfp4", 0, 0, 1)


def test_dual_4096x4096_m1():
    _run("rocmfp4_dual", 1, 0, 1)


def test_decode_sweep_one_layer():
    # the seven shapes of one 4B-class layer (the sweep repeats them 36 times)
    for mat in range(7):
        _run("nvfp4", 2, mat, 1)


@pytest.mark.parametrize("fmt", ["nvfp4", "rocmfp4_dual", "rocmfp4_fast", "q4_0"])
@pytest.mark.parametrize("m", [1, 4, 6, 9, 16, 33, 64])
def test_spec_verify(fmt, m):
    if fmt == "q4_0" and m > 16:
        pytest.skip("Q4_0 runs through the GEMV only (M <= 16)")
    for mat in range(2):
        _run(fmt, 3, mat, m)


@pytest.mark.parametrize("fmt", ["rocmfp4_fast", "nvfp4"])
def test_prefill_m2048(fmt):
    rng = np.random.default_rng(60)
    n = synth.WORKLOADS[4]["shapes"][0][0]
    cols = np.unique(np.concatenate([[0, 1, 15, 16, 127, 128, n - 1], rng.choice(n, 57, replace=False)]))
    _run(fmt, 4, 0, 2048, cols=cols)


def test_decode_sweep_layer_grouped_launches():
    # one 4B-class layer at full size through the launch patterns the sweep benchmark times: q|k|v as
    # one grouped launch on one x, o alone, gate|up as one grouped launch on one x, down alone; then
    # the same seven products as one device-list launch. Every output column against the oracle.
    fmt, cfg = "nvfp4", 2
    shapes = synth.WORKLOADS[cfg]["shapes"][:7]
    print("CASE decode-sweep layer grouped launches", shapes, flush=True)
    packed, pws = [], []
    for mat, (n, k) in enumerate(shapes):
        p = pack.pack(fmt, synth.workload_weights(cfg, mat))
        packed.append(p)
        pws.append(gc.upload(fmt, n, k, p))
    # one x per consumer: q, k and v read the same x, so do gate and up
    x_of = (0, 0, 0, 3, 4, 4, 6)
    xb = {j: synth.workload_activations(cfg, j, 1) for j in set(x_of)}
    xt = {j: gc.x_tensor(v) for j, v in xb.items()}
    for label, groups in (("decode order", ((0, 1, 2), (3,), (4, 5), (6,))), ("device list", (tuple(range(7)),))):
        ys = [torch.full((1, n), float("nan"), device="cuda") for (n, _) in shapes]
        for grp in groups:
            fp4.w4a16_gemv_batched(fmt, 1, [(pws[i].q, pws[i].s, pws[i].global_scale, xt[x_of[i]], ys[i],
                                             shapes[i][0], shapes[i][1]) for i in grp])
        torch.cuda.synchronize()
        for i, (n, k) in enumerate(shapes):
            gc.check_product(fmt, packed[i], xb[x_of[i]], ys[i], label=f"{label} {n}x{k}")
