"""Packers that turn fp32 weights into canonical packed bytes (CPU oracle, FP64 decisions).

NVFP4 - data-free round-to-nearest (Nanbeige4.2-3B-NVFP4A16 card, "Creation": the
NVFP4A16 scheme applied data-free, i.e. RTN; EdgeRock-4B-NVFP4 card: E2M1 codes,
an E4M3 byte for each group of 16 weights, one FP32 factor for the matrix):
  1. amax = max |W|; g = fl32(amax / (6 * 448))  (the global scale maps the largest
     block scale to the E4M3 maximum 448 and the largest weight to E2M1's 6);
  2. per 16-weight block: s = E4M3 RNE of max|w_block| / (6 g)  (FP64 divide);
  3. d = e4m3(s) * g; each weight takes the E2M1 magnitude nearest |w| / d, decided by
     exact comparison of |w| with the midpoints {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5} d,
     ties to the even code, above 5 d -> 6; the sign bit is set iff w < 0 and the
     magnitude is nonzero.
  Readings: amax = 0 (or g underflowing to 0) packs all-zero codes with g = 1; d = 0
  gives zero codes for the block.

ROCmFP4 - exhaustive finite-UE4M3 MSE search per scale group (ROCmFP4 design page,
section 03); see csrc/rocmfp4_search.c for the steps and readings. g = 1.

Q4_0 - signed abs-max scale (ROCmFP4 design page, comparison table: the stock Q4_0
reference scale is derived from the signed abs-max; no imatrix):
  1. per 32-weight block, m = the weight of largest magnitude, keeping its sign (the
     first one in index order on a tie of magnitudes); d = m / -8 (exact in FP64), so
     that m lands on the grid's -8 end;
  2. the stored scale is d rounded to FP16 (RNE);
  3. each code is the grid point nearest w / d rounding halves up, q = floor(w / d + 8.5)
     clipped to 0..15, decided in FP64 with the unrounded d (exact: w / d is a ratio of
     FP32 values scaled by 8); d = 0 (an all-zero block) gives code 8 (level 0).
  Readings: which d decides the codes and the tie rule are not on the pages; the
  stored scale is what dequantisation uses. g = 1.

Return shapes: NVFP4 -> (wq u8[N, K/2], ws u8[N, K/16], g float32);
ROCmFP4 and Q4_0 -> (blocks u8[N, K/32, 18 | 17], g = float32(1)).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build
from . import formats, layouts

E2M1_MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float64)

_lib = None


def _clib():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        lib = ctypes.CDLL(path)
        lib.oracle_rocmfp4_search.restype = ctypes.c_int
        lib.oracle_rocmfp4_search.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                              ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p]
        lib.oracle_rocmfp4_all_errors.restype = ctypes.c_int
        lib.oracle_rocmfp4_all_errors.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                                  ctypes.c_int, ctypes.c_void_p]
        _lib = lib
    return _lib


def _nearest_code(a: np.ndarray, d: np.ndarray, midpoints: np.ndarray) -> np.ndarray:
    """Magnitude code of the level nearest a/d: count the midpoints*d strictly below a,
    then move an exact tie on an odd code up to the even neighbour. a, d: same shape."""
    code = np.zeros(a.shape, dtype=np.int64)
    for t in midpoints:
        code += a > t * d                                 # t * d is exact
    at_c = midpoints[np.minimum(code, len(midpoints) - 1)] * d
    tie = (code < len(midpoints)) & (a == at_c) & (code % 2 == 1)
    return (code + tie).astype(np.uint8)


def _nvfp4_rows(w: np.ndarray, g: np.float32):
    """Steps 2-3 on a slab of rows, given the matrix's global scale g."""
    n, k = w.shape
    a = np.abs(w.astype(np.float64)).reshape(n * (k // 16), 16)
    scale_codes = formats.e4m3_encode_rne(a.max(axis=1) / (6.0 * np.float64(g)))
    d = formats.e4m3_value(scale_codes) * np.float64(g)
    mag = np.zeros(a.shape, dtype=np.uint8)
    nz = d > 0
    if np.any(nz):
        mag[nz] = _nearest_code(a[nz], np.broadcast_to(d[nz][:, None], a[nz].shape), E2M1_MIDPOINTS)
    neg = (w.reshape(a.shape) < 0) & (mag != 0)
    codes = (mag | (neg.astype(np.uint8) << 3)).reshape(n, k)
    return layouts.nvfp4_join(codes), scale_codes.reshape(n, k // 16)


def nvfp4_global_scale(w: np.ndarray) -> np.float32:
    """Step 1: g = fl32(amax / 2688) of the whole matrix (0 when amax is 0)."""
    w = np.asarray(w, dtype=np.float32)
    amax = np.float32(np.max(np.abs(w))) if w.size else np.float32(0)
    return np.float32(amax) / np.float32(6 * 448) if amax > 0 else np.float32(0)


def pack_nvfp4_rows(w_rows: np.ndarray, g: np.float32, rows_per_slab: int = 512):
    """Steps 2-3 for some rows of a matrix whose global scale g (step 1, over the whole matrix) is
    given: rows are packed independently once g is known, so a row sample packs to exactly the bytes
    those rows get in the whole matrix."""
    w = np.ascontiguousarray(w_rows, dtype=np.float32)
    n, k = w.shape
    if k % layouts.NVFP4_GROUP:
        raise ValueError("K must be a multiple of 16 for NVFP4")
    if not (g > 0):
        return (np.zeros((n, k // 2), np.uint8), np.zeros((n, k // 16), np.uint8), np.float32(1.0))
    wq = np.empty((n, k // 2), np.uint8)
    ws = np.empty((n, k // 16), np.uint8)
    for r0 in range(0, n, rows_per_slab):
        wq[r0:r0 + rows_per_slab], ws[r0:r0 + rows_per_slab] = _nvfp4_rows(w[r0:r0 + rows_per_slab], g)
    return (wq, ws, np.float32(g))


def pack_nvfp4(w: np.ndarray, rows_per_slab: int = 512):
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.shape[1] % layouts.NVFP4_GROUP:
        raise ValueError("K must be a multiple of 16 for NVFP4")
    return pack_nvfp4_rows(w, nvfp4_global_scale(w), rows_per_slab)


def rocmfp4_search(w_groups: np.ndarray, importance: np.ndarray | None = None):
    """Search every row of w_groups [G, group]; returns (codes u8[G, group], scales u8[G], errs f64[G])."""
    w = np.ascontiguousarray(w_groups, dtype=np.float32)
    ng, group = w.shape
    v = None if importance is None else np.ascontiguousarray(importance, dtype=np.float32)
    if v is not None and v.shape != w.shape:
        raise ValueError("importance must match the weights' shape")
    codes = np.empty((ng, group), dtype=np.uint8)
    scales = np.empty(ng, dtype=np.uint8)
    errs = np.empty(ng, dtype=np.float64)
    rc = _clib().oracle_rocmfp4_search(w.ctypes.data, None if v is None else v.ctypes.data, ng, group,
                                       codes.ctypes.data, scales.ctypes.data, errs.ctypes.data)
    if rc != 0:
        raise ValueError("bad group size")
    return codes, scales, errs


def rocmfp4_all_errors(w_groups: np.ndarray, importance: np.ndarray | None = None) -> np.ndarray:
    """E(c) for all 127 candidates: f64[G, 127]."""
    w = np.ascontiguousarray(w_groups, dtype=np.float32)
    ng, group = w.shape
    v = None if importance is None else np.ascontiguousarray(importance, dtype=np.float32)
    errs = np.empty((ng, formats.UE4M3_FINITE_CODES), dtype=np.float64)
    _clib().oracle_rocmfp4_all_errors(w.ctypes.data, None if v is None else v.ctypes.data, ng, group,
                                      errs.ctypes.data)
    return errs


def pack_rocmfp4(fmt: str, w: np.ndarray, importance: np.ndarray | None = None):
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    if k % layouts.ROCM_BLOCK:
        raise ValueError("K must be a multiple of 32 for ROCmFP4")
    group = layouts.scale_group(fmt)
    codes, scales, _ = rocmfp4_search(w.reshape(-1, group),
                                      None if importance is None else np.asarray(importance).reshape(-1, group))
    blocks = layouts.rocm_join(fmt, codes.reshape(n, k), scales.reshape(n, -1))
    return (blocks, np.float32(1.0))


def pack_q4_0(w: np.ndarray):
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    if k % layouts.ROCM_BLOCK:
        raise ValueError("K must be a multiple of 32 for Q4_0")
    b = w.astype(np.float64).reshape(n * (k // 32), 32)
    first = np.argmax(np.abs(b), axis=1)                  # first index of the largest magnitude
    m = b[np.arange(b.shape[0]), first]
    d = m / -8.0 + 0.0                                    # + 0.0: an all-zero block stores +0
    d_bits = formats.fp16_encode_rne(d)
    safe = np.where(d != 0.0, d, 1.0)
    q = np.floor(b / safe[:, None] + 8.5)
    q = np.where((d != 0.0)[:, None], np.clip(q, 0, 15), 8).astype(np.uint8)
    return (layouts.q4_0_join(q.reshape(n, k), d_bits.reshape(n, k // 32)), np.float32(1.0))


def pack(fmt: str, w: np.ndarray, importance: np.ndarray | None = None):
    if fmt in ("nvfp4", "q4_0"):
        if importance is not None:
            raise ValueError(f"the {fmt} packer takes no importance")
        return pack_nvfp4(w) if fmt == "nvfp4" else pack_q4_0(w)
    return pack_rocmfp4(fmt, w, importance)
