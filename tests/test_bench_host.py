"""Host-side logic of bench.py (CPU only): algorithmic byte counts, the stale-counter rule, --gpus."""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_match_the_format_densities():
    # 4.5 bits per weight for NVFP4 (4-bit code + one 8-bit scale per 16) and Dual (18 B per 32 weights),
    # 4.25 for FAST (17 B per 32)
    assert bench.algorithmic_bytes("nvfp4", 2048, 2048) == 2048 * 2048 * 9 // 16 == 2_359_296
    assert bench.algorithmic_bytes("rocmfp4_dual", 4096, 4096) == 4096 * 128 * 18 == 9_437_184
    assert bench.algorithmic_bytes("rocmfp4_fast", 14336, 4096) == 14336 * 128 * 17 == 31_195_136
    assert bench.algorithmic_bytes("nvfp4", 14336, 4096) == 33_030_144
    assert bench.algorithmic_bytes("rocmfp4_dual", 9728, 2560) == bench.algorithmic_bytes("nvfp4", 9728, 2560)
    assert bench.algorithmic_bytes("rocmfp4_fast", 9728, 2560) == 9728 * 80 * 17


def test_decode_sweep_bytes():
    # 36 layers of q, k, v, o, gate, up, down in NVFP4
    total = sum(bench.algorithmic_bytes("nvfp4", n, k) for (n, k) in synth.WORKLOADS[2]["shapes"])
    assert len(synth.WORKLOADS[2]["shapes"]) == 252
    assert total == 36 * (2 * 5_898_240 + 2 * 1_474_560 + 3 * 14_008_320) == 2_043_740_160


def test_traffic_is_dropped_when_the_kernel_source_changed(monkeypatch):
    # a counter figure is reported only while the kernel source it was taken on is unchanged
    real = bench.kernel_source_hash("gemv.hip")
    got = bench.traffic_from_profiles("gemv.hip", "rocmfp4_dual_4096x4096_m1")
    monkeypatch.setattr(bench, "kernel_source_hash", lambda name: real[::-1])
    assert bench.traffic_from_profiles("gemv.hip", "rocmfp4_dual_4096x4096_m1") is None
    monkeypatch.undo()
    if got is not None:
        assert 9_437_184 <= got < 2 * 9_437_184
    assert bench.traffic_from_profiles("gemv.hip", "no_such_workload") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout


def test_oracle_sample_gate_passes_the_oracle_and_fails_a_perturbed_output():
    # the parity gate of the CPU-baseline leg: the oracle's own product passes, a product with one
    # element off by more than the tolerance is flagged (so that workload's throughput is withheld)
    from oracle import pack, ref
    w = synth.weights(64, 256, dist="t", nu=5.0, cfg=95)
    x_bits = synth.activations(3, 256, cfg=95, mat=1)
    for fmt in ("nvfp4", "rocmfp4_dual", "rocmfp4_fast"):
        y = ref.matmul(x_bits, ref.dequant(fmt, pack.pack(fmt, w))).astype(np.float32)
        rows = bench.sample_rows(64, 16)
        good = bench.oracle_sample(fmt, w, rows, x_bits, y, threads=3, budget_s=0.0)
        assert good["parity"] and good["rows"] == len(rows) and good["runs"] >= 3
        bad_y = y.copy()
        bad_y[1, rows[5]] += 0.5
        assert not bench.oracle_sample(fmt, w, rows, x_bits, bad_y, threads=2, budget_s=0.0, time_it=False)["parity"]


def test_sample_rows_cover_both_ends():
    r = bench.sample_rows(4096, 512)
    assert r[0] == 0 and r[-1] == 4095 and len(r) == 512 and np.all(np.diff(r) > 0)
    assert list(bench.sample_rows(5, 512)) == [0, 1, 2, 3, 4]
