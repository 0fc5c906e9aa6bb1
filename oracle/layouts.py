"""Canonical byte layouts of the packed weights, and their sizes.

Sources:
* EdgeRock-4B-NVFP4 model card (description; package section): an NVFP4
  matrix is stored as 4-bit codes, an E4M3 byte for every group of 16 weights
  and a single FP32 factor for the whole matrix.
* ROCmFP4 design page, format comparison table: 32 weights per block; Dual
  carries two UE4M3 bytes (one per 16-weight half) in 18 bytes = 4.50 bits per
  weight; FAST carries one UE4M3 byte in 17 bytes = 4.25 bits per weight; stock
  Q4_0 carries one FP16 scale in 18 bytes = 4.50 bits per weight.

Readings (no byte order is printed on the pages):
* NVFP4: wq u8[N][K/2], byte j of a row holds element 2j in bits 0-3 and element
  2j+1 in bits 4-7; ws u8[N][K/16]; g is one float32.
* ROCmFP4 (a Q4_0 derivative, whose two-byte scale field becomes the scale
  bytes): row n is K/32 consecutive blocks. Dual = [s_lo, s_hi, qs[16]],
  FAST = [s, qs[16]]; qs[j] holds weight j in its low nibble and weight j+16 in
  its high nibble. In Dual, weights 0..15 use s_lo and 16..31 use s_hi.
* Q4_0: the same 16 nibble bytes after a little-endian FP16 scale:
  [d_lo, d_hi, qs[16]].
"""
from __future__ import annotations

import numpy as np

NVFP4_GROUP = 16
ROCM_BLOCK = 32
BLOCK_BYTES = {"rocmfp4_dual": 18, "rocmfp4_fast": 17, "q4_0": 18}
SCALES_PER_BLOCK = {"rocmfp4_dual": 2, "rocmfp4_fast": 1}
BLOCK_FORMATS = ("rocmfp4_dual", "rocmfp4_fast", "q4_0")


def k_multiple(fmt: str) -> int:
    return NVFP4_GROUP if fmt == "nvfp4" else ROCM_BLOCK


def canonical_bytes(fmt: str, n: int, k: int) -> int:
    """Bytes of the canonical packed matrix (weights + scales; NVFP4's g excluded)."""
    if k % k_multiple(fmt):
        raise ValueError(f"K={k} is not a multiple of {k_multiple(fmt)} for {fmt}")
    if fmt == "nvfp4":
        return n * (k // 2 + k // NVFP4_GROUP)
    return n * (k // ROCM_BLOCK) * BLOCK_BYTES[fmt]


def bits_per_weight(fmt: str) -> float:
    k = 32 * NVFP4_GROUP
    return 8.0 * canonical_bytes(fmt, 1, k) / k


# ----------------------------------------------------------------------------
# Code/scale planes <-> canonical bytes. "codes" are nibbles as uint8 [N, K]
# (element order), "scale_codes" are the scale bytes, one per scale group in
# element order: [N, K/16] for NVFP4 and Dual, [N, K/32] for FAST.
# ----------------------------------------------------------------------------

def nvfp4_split(wq: np.ndarray) -> np.ndarray:
    """wq u8[N, K/2] -> codes u8[N, K]."""
    wq = np.asarray(wq, dtype=np.uint8)
    n, half = wq.shape
    codes = np.empty((n, 2 * half), dtype=np.uint8)
    codes[:, 0::2] = wq & 0x0F
    codes[:, 1::2] = wq >> 4
    return codes


def nvfp4_join(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] & 0x0F) | ((codes[:, 1::2] & 0x0F) << 4)


def rocm_split(fmt: str, blocks: np.ndarray):
    """blocks u8[N, K/32, B] -> (codes u8[N, K], scale_codes u8[N, K/32 * scales_per_block])."""
    blocks = np.asarray(blocks, dtype=np.uint8)
    n, nb, bb = blocks.shape
    if bb != BLOCK_BYTES[fmt]:
        raise ValueError(f"{fmt} blocks are {BLOCK_BYTES[fmt]} bytes, got {bb}")
    ns = SCALES_PER_BLOCK[fmt]
    qs = blocks[:, :, ns:]                      # [N, nb, 16]
    codes = np.empty((n, nb, ROCM_BLOCK), dtype=np.uint8)
    codes[:, :, :16] = qs & 0x0F
    codes[:, :, 16:] = qs >> 4
    scale_codes = blocks[:, :, :ns].reshape(n, nb * ns)
    return codes.reshape(n, nb * ROCM_BLOCK), scale_codes.copy()


def rocm_join(fmt: str, codes: np.ndarray, scale_codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    n, k = codes.shape
    nb = k // ROCM_BLOCK
    ns = SCALES_PER_BLOCK[fmt]
    c = codes.reshape(n, nb, ROCM_BLOCK)
    out = np.empty((n, nb, BLOCK_BYTES[fmt]), dtype=np.uint8)
    out[:, :, :ns] = np.asarray(scale_codes, dtype=np.uint8).reshape(n, nb, ns)
    out[:, :, ns:] = (c[:, :, :16] & 0x0F) | ((c[:, :, 16:] & 0x0F) << 4)
    return out


def q4_0_split(blocks: np.ndarray):
    """Q4_0 blocks u8[N, K/32, 18] -> (codes u8[N, K], scale bits u16[N, K/32])."""
    blocks = np.asarray(blocks, dtype=np.uint8)
    n, nb, bb = blocks.shape
    if bb != BLOCK_BYTES["q4_0"]:
        raise ValueError(f"q4_0 blocks are 18 bytes, got {bb}")
    qs = blocks[:, :, 2:]
    codes = np.empty((n, nb, ROCM_BLOCK), dtype=np.uint8)
    codes[:, :, :16] = qs & 0x0F
    codes[:, :, 16:] = qs >> 4
    d_bits = blocks[:, :, 0].astype(np.uint16) | (blocks[:, :, 1].astype(np.uint16) << 8)
    return codes.reshape(n, nb * ROCM_BLOCK), d_bits


def q4_0_join(codes: np.ndarray, d_bits: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    n, k = codes.shape
    nb = k // ROCM_BLOCK
    c = codes.reshape(n, nb, ROCM_BLOCK)
    d = np.asarray(d_bits, dtype=np.uint16).reshape(n, nb)
    out = np.empty((n, nb, 18), dtype=np.uint8)
    out[:, :, 0] = d & 0xFF
    out[:, :, 1] = d >> 8
    out[:, :, 2:] = (c[:, :, :16] & 0x0F) | ((c[:, :, 16:] & 0x0F) << 4)
    return out


def scale_group(fmt: str) -> int:
    """Number of consecutive weights sharing one scale."""
    return 16 if fmt in ("nvfp4", "rocmfp4_dual") else 32
