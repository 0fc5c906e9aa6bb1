"""Exact dequantisation and the FP64 reference product.

Definition followed (EdgeRock-4B-NVFP4 model card, description; ROCmFP4 design
page, sections 01-02 and the comparison table):

    NVFP4:         W[n, k] = e2m1(q[n, k]) * e4m3(ws[n, k // 16]) * g
    ROCmFP4 Dual:  W[n, 32b + j] = codebook10(q) * ue4m3(s[b][j >= 16])
    ROCmFP4 FAST:  W[n, 32b + j] = codebook10(q) * ue4m3(s[b])
    Q4_0:          W[n, 32b + j] = (q - 8) * fp16(d[b])          (comparison table, stock Q4_0)
    y[m, n] = sum_k x[m, k] * W[n, k]          (x is bf16, y is reported in fp32)

Readings:
* The pages list the three NVFP4 factors but no order of multiplication. In FP64
  every product above is exact (at most 3 + 4 + 24 significant bits), so the
  oracle's W is the exact product. The bit-exact FP32 dequant target is one
  round-to-nearest-even of that exact value.
* The pages list no tensor-level scale for ROCmFP4 or Q4_0 (the block metadata is
  the scale bytes only), so g = 1 there; the interface still takes g.

Acceptance (the tolerance of the GPU path): |y_gpu - y_ref| <= 2e-3 * B + 1e-6 with
B[m, n] = sum_k |x[m, k] * W[n, k]|.
"""
from __future__ import annotations

import numpy as np

from . import formats, layouts

REL_TOL = 2e-3
ABS_TOL = 1e-6


def bf16_bits_to_f64(x_bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact FP64 values."""
    u = np.asarray(x_bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def dequant_nvfp4(wq: np.ndarray, ws: np.ndarray, g: float) -> np.ndarray:
    codes = layouts.nvfp4_split(wq)
    n, k = codes.shape
    level = formats.e2m1_value(codes)
    scale = np.repeat(formats.e4m3_value(ws), layouts.NVFP4_GROUP, axis=1)
    assert scale.shape == (n, k)
    return level * scale * np.float64(np.float32(g))


def dequant_rocmfp4(fmt: str, blocks: np.ndarray, g: float = 1.0) -> np.ndarray:
    codes, scale_codes = layouts.rocm_split(fmt, blocks)
    level = formats.codebook10_value(codes)
    scale = np.repeat(formats.ue4m3_value(scale_codes), layouts.scale_group(fmt), axis=1)
    return level * scale * np.float64(np.float32(g))


def dequant_q4_0(blocks: np.ndarray, g: float = 1.0) -> np.ndarray:
    codes, d_bits = layouts.q4_0_split(blocks)
    level = formats.q4_0_value(codes)
    scale = np.repeat(formats.fp16_value(d_bits), layouts.ROCM_BLOCK, axis=1)
    return level * scale * np.float64(np.float32(g))


def dequant(fmt: str, packed) -> np.ndarray:
    """Exact FP64 W[N, K] from a packed matrix (see pack.py for the tuple shapes)."""
    if fmt == "nvfp4":
        wq, ws, g = packed
        return dequant_nvfp4(wq, ws, g)
    blocks, g = packed
    if fmt == "q4_0":
        return dequant_q4_0(blocks, g)
    return dequant_rocmfp4(fmt, blocks, g)


def dequant_f32(fmt: str, packed) -> np.ndarray:
    """The bit-exact FP32 target: a single RNE rounding of the exact value."""
    return dequant(fmt, packed).astype(np.float32)


def matmul(x_bits: np.ndarray, w64: np.ndarray) -> np.ndarray:
    """y = x W^T in FP64 (x given as bf16 bit patterns [M, K], W as FP64 [N, K])."""
    return bf16_bits_to_f64(x_bits) @ w64.T


def bound(x_bits: np.ndarray, w64: np.ndarray) -> np.ndarray:
    """B[m, n] = sum_k |x[m, k] W[n, k]|, the scale of the tolerance."""
    return np.abs(bf16_bits_to_f64(x_bits)) @ np.abs(w64).T


def rows(fmt: str, packed, idx) -> tuple:
    """Restrict a packed matrix to output rows `idx` (for sampled checks at full size)."""
    idx = np.asarray(idx)
    if fmt == "nvfp4":
        wq, ws, g = packed
        return (wq[idx], ws[idx], g)
    blocks, g = packed
    return (blocks[idx], g)


def check(y_gpu: np.ndarray, y_ref: np.ndarray, b: np.ndarray):
    """Elementwise acceptance; returns (ok, worst ratio of error to allowance)."""
    err = np.abs(np.asarray(y_gpu, dtype=np.float64) - y_ref)
    allow = REL_TOL * b + ABS_TOL
    ratio = err / allow
    worst = float(np.nanmax(ratio)) if ratio.size else 0.0
    ok = bool(np.all(err <= allow)) and not np.any(np.isnan(y_gpu))
    return ok, worst
