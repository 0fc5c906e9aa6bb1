"""Seeded synthetic inputs shared by the CPU oracle's tests and the GPU path.

This module only draws random numbers. It holds none of the W4A16 arithmetic:
no codec, no packing, no dequantisation, no product. Weights come out as fp32
arrays, activations as bf16 bit patterns (uint16), and raw canonical bytes as
uint8 arrays with a stated value range.

Seeding: every stream is ``numpy.random.Generator(PCG64(SeedSequence(ROOT_SEED,
spawn_key=(cfg, mat, stream))))``. ``cfg`` names the workload, ``mat`` the
matrix inside it, ``stream`` what is drawn (0 weights, 1 outlier positions,
2 activations, 3 raw bytes).

The distributions follow the decode and prefill workloads the pages describe:
Student-t or normal weights scaled by 0.02 (the spread of a 4B-class
transformer's linear layers), optional 0.1 % outliers at 20x, and N(0, 1)
activations rounded to bf16.
"""
from __future__ import annotations

import numpy as np

ROOT_SEED = 20261203

STREAM_W = 0
STREAM_OUTLIER = 1
STREAM_X = 2
STREAM_BYTES = 3


def rng(cfg: int, mat: int, stream: int) -> np.random.Generator:
    """Independent PCG64 stream for (workload, matrix, purpose)."""
    ss = np.random.SeedSequence(ROOT_SEED, spawn_key=(int(cfg), int(mat), int(stream)))
    return np.random.Generator(np.random.PCG64(ss))


def weights(n: int, k: int, *, dist: str = "normal", nu: float = 5.0, sigma: float = 0.02,
            outlier_frac: float = 0.0, outlier_mult: float = 20.0,
            cfg: int = 0, mat: int = 0) -> np.ndarray:
    """fp32 weights W[n, k] (n outputs, k inputs).

    dist: "normal" -> N(0, sigma^2); "t" -> Student-t(nu) * sigma.
    outlier_frac > 0 picks round(frac*n*k) distinct positions and multiplies them
    by outlier_mult.
    """
    g = rng(cfg, mat, STREAM_W)
    if dist == "normal":
        w = g.normal(0.0, sigma, size=(n, k))
    elif dist == "t":
        w = g.standard_t(nu, size=(n, k)) * sigma
    else:
        raise ValueError(f"unknown weight distribution {dist!r}")
    w = w.astype(np.float32)
    if outlier_frac > 0.0:
        count = int(round(outlier_frac * n * k))
        pos = rng(cfg, mat, STREAM_OUTLIER).choice(n * k, size=count, replace=False)
        flat = w.reshape(-1)
        flat[pos] = flat[pos] * np.float32(outlier_mult)
    return w


def device_weights(n: int, k: int, *, sigma: float = 0.02, cfg: int = 0, mat: int = 0, device="cuda"):
    """N(0, sigma^2) fp32 weights W[n, k] drawn on a torch device (for benchmark-sized workloads).

    Same recipe as ``weights(dist="normal")``, drawn by torch's generator for ``device`` seeded from
    the (cfg, mat) weight stream, so a many-GB workload is generated in place in seconds. The values
    differ from the numpy draw of the same (cfg, mat); tests that compare with the oracle use
    ``weights``.
    """
    import torch
    seed = int(np.random.SeedSequence(ROOT_SEED, spawn_key=(int(cfg), int(mat), STREAM_W)).generate_state(1)[0])
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn((n, k), generator=g, device=device, dtype=torch.float32) * sigma


def _f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest bf16 (ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def activations(m: int, k: int, *, cfg: int = 0, mat: int = 0, scale: float = 1.0) -> np.ndarray:
    """bf16 activations x[m, k] drawn from N(0, scale^2), as uint16 bit patterns."""
    g = rng(cfg, mat, STREAM_X)
    x = (g.standard_normal(size=(m, k)) * scale).astype(np.float32)
    return _f32_to_bf16_bits(x)


def raw_bytes(shape, *, low: int = 0, high: int = 256, cfg: int = 0, mat: int = 0) -> np.ndarray:
    """Uniform random bytes in [low, high) — used for arbitrary (not fitted) packed codes."""
    g = rng(cfg, mat, STREAM_BYTES)
    return g.integers(low, high, size=shape, dtype=np.int64).astype(np.uint8)


# ---------------------------------------------------------------------------
# The workloads. Shapes are (N out, K in). Each entry names the weight draw so
# that every layout run on a workload packs the same fp32 matrix.
# ---------------------------------------------------------------------------

DECODE_4B_LAYER = (  # one layer of a 4B-class decoder: hidden 2560, 16x256 q heads, 4x256 kv heads
    ("q", 4096, 2560), ("k", 1024, 2560), ("v", 1024, 2560), ("o", 2560, 4096),
    ("gate", 9728, 2560), ("up", 9728, 2560), ("down", 2560, 9728),
)

WORKLOADS = {
    # cfg id: description
    0: dict(name="nvfp4_2048x2048_m1", fmt=("nvfp4",), shapes=[(2048, 2048)], ms=(1,),
            dist="t", nu=5.0, outlier_frac=0.0),
    1: dict(name="rocmfp4_dual_4096x4096_m1", fmt=("rocmfp4_dual",), shapes=[(4096, 4096)], ms=(1,),
            dist="t", nu=4.0, outlier_frac=0.001),
    2: dict(name="nvfp4_4b_decode_sweep_m1", fmt=("nvfp4",),
            shapes=[(n, k) for _ in range(36) for (_, n, k) in DECODE_4B_LAYER], ms=(1,),
            dist="normal", nu=0.0, outlier_frac=0.0),
    3: dict(name="spec_verify_9728x2560_2560x9728", fmt=("nvfp4", "rocmfp4_dual", "rocmfp4_fast"),
            shapes=[(9728, 2560), (2560, 9728)], ms=(1, 9, 16),
            dist="t", nu=5.0, outlier_frac=0.0),
    4: dict(name="prefill_m2048_k4096_n14336", fmt=("rocmfp4_fast", "nvfp4"), shapes=[(14336, 4096)],
            ms=(2048,), dist="normal", nu=0.0, outlier_frac=0.0),
}


def workload_weights(cfg: int, mat: int) -> np.ndarray:
    """fp32 weights of matrix `mat` of workload `cfg`."""
    w = WORKLOADS[cfg]
    n, k = w["shapes"][mat]
    return weights(n, k, dist=w["dist"], nu=w["nu"], outlier_frac=w["outlier_frac"], cfg=cfg, mat=mat)


def workload_activations(cfg: int, mat: int, m: int) -> np.ndarray:
    w = WORKLOADS[cfg]
    _, k = w["shapes"][mat]
    return activations(m, k, cfg=cfg, mat=1000 * m + mat)
