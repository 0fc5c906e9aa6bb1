"""Python binding of the fp4w4a16 C ABI (block-scaled 4-bit weights x bf16 activations on gfx950).

Argument marshalling only: every function below checks tensor devices, dtypes and sizes,
passes raw device pointers and the current HIP stream to the C entry point of the same
name in libfp4w4a16.so, and raises RuntimeError on a negative status. All computation
runs in the library's HIP kernels; there is no fallback path. Importing this package
without the built library fails loudly.
"""
from __future__ import annotations

import ctypes
import functools
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp4w4a16.so")

FORMATS = {"nvfp4": 1, "rocmfp4_dual": 2, "rocmfp4_fast": 3, "q4_0": 4}
BLOCK_BYTES = {"rocmfp4_dual": 18, "rocmfp4_fast": 17, "q4_0": 18}
GEMV_MAX_M = 16

_c = ctypes.c_int
_i64 = ctypes.c_int64
_p = ctypes.c_void_p
_f = ctypes.c_float

GEMV_MAX_ITEMS = 32


class GemvItem(ctypes.Structure):
    """Mirror of `fp4_gemv_item` (one matrix of a w4a16_gemv_batched call)."""
    _fields_ = [("q", ctypes.c_void_p), ("s", ctypes.c_void_p), ("x_bf16", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("global_scale", ctypes.c_float)]


_SIGS = {
    "fp4_abi_version": (_c, []),
    "fp4_status_string": (ctypes.c_char_p, [_c]),
    "fp4_layout_bytes": (_c, [_c, _i64, _i64, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]),
    "fp4_pack_layout": (_c, [_c, _i64, _i64, _p, _p, _p, _p, _c, _p]),
    "w4a16_gemv": (_c, [_c, _i64, _i64, _i64, _p, _p, _f, _p, _p, _p]),
    "w4a16_gemv_batched": (_c, [_c, _i64, _c, ctypes.POINTER(GemvItem), _p]),
    "w4a16_gemm": (_c, [_c, _i64, _i64, _i64, _p, _p, _f, _p, _p, _p]),
    "w4a16_midm": (_c, [_c, _i64, _i64, _i64, _p, _p, _f, _p, _p, _p]),
    "w4a16_matmul": (_c, [_c, _i64, _i64, _i64, _p, _p, _f, _p, _p, _p]),
    "w4a16_gemm_ws": (_c, [_c, _i64, _i64, _i64, _p, _p, _f, _p, _p, _p, ctypes.c_size_t, _p]),
    "w4a16_matmul_ws": (_c, [_c, _i64, _i64, _i64, _p, _p, _f, _p, _p, _p, ctypes.c_size_t, _p]),
    "w4a16_gemm_workspace_bytes": (_i64, [_c, _i64, _i64, _i64]),
    "w4a16_matmul_workspace_bytes": (_i64, [_c, _i64, _i64, _i64]),
    "w4a16_gemm_noalloc": (_c, [_c, _i64, _i64, _i64, _p, _p, _f, _p, _p, _p]),
    "fp4_dequant_f32": (_c, [_c, _i64, _i64, _p, _p, _f, _p, _p]),
    "fp4_quantize_nvfp4": (_c, [_i64, _i64, _p, _p, _p, _p, _p]),
    "fp4_quantize_rocmfp4": (_c, [_c, _i64, _i64, _p, _p, _p, _p]),
    "fp4_quantize_q4_0": (_c, [_i64, _i64, _p, _p, _p]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with block_scaled_fp4_w4a16_amd/build.py "
                              "(or __graft_entry__.build())")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


lib()  # fail at import time when the HIP library is absent


def _fmt(fmt) -> int:
    if isinstance(fmt, str):
        if fmt not in FORMATS:
            raise ValueError(f"unknown format {fmt!r}; expected one of {sorted(FORMATS)}")
        return FORMATS[fmt]
    return int(fmt)


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what}: {lib().fp4_status_string(rc).decode()} (status {rc})")


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _device(*ts) -> torch.device:
    """The one GPU that every given tensor (None entries skipped) lives on; the call runs there."""
    devs = {t.device for t in ts if isinstance(t, torch.Tensor)}
    if len(devs) != 1:
        raise ValueError(f"tensors must all live on one GPU (got {sorted(str(d) for d in devs)})")
    d = devs.pop()
    if d.type != "cuda":
        raise ValueError("tensors must live on the GPU")
    return d


@functools.lru_cache(maxsize=4096)
def _plane_bytes(f: int, N: int, K: int) -> tuple[int, int]:
    q = ctypes.c_size_t()
    s = ctypes.c_size_t()
    _check(lib().fp4_layout_bytes(f, N, K, ctypes.byref(q), ctypes.byref(s)), "fp4_layout_bytes")
    return q.value, s.value


def _check_planes(f: int, N: int, K: int, q, s):
    qb, sb = _plane_bytes(f, N, K)
    if _nbytes(q) < qb or _nbytes(s) < sb:
        raise ValueError(f"packed planes too small for N={N} K={K}: need {qb} + {sb} bytes, "
                         f"got {_nbytes(q)} + {_nbytes(s)}")


def fp4_abi_version() -> int:
    return lib().fp4_abi_version()


def fp4_status_string(status: int) -> str:
    return lib().fp4_status_string(status).decode()


def fp4_layout_bytes(fmt, N: int, K: int) -> tuple[int, int]:
    q = ctypes.c_size_t()
    s = ctypes.c_size_t()
    _check(lib().fp4_layout_bytes(_fmt(fmt), N, K, ctypes.byref(q), ctypes.byref(s)), "fp4_layout_bytes")
    return q.value, s.value


def fp4_pack_layout(fmt, N, K, src_q, src_s, dst_q, dst_s, validate=False, stream=None):
    """Canonical bytes -> kernel layout. validate=True first checks every scale code on the device
    (waits for the stream) and raises RuntimeError with the library's FP4_ERR_INVALID_SCALE status,
    leaving dst_q / dst_s untouched, if one is NaN (or, for Q4_0, not finite)."""
    f = _fmt(fmt)
    dev = _device(src_q, src_s, dst_q, dst_s)
    if N > 0 and K > 0 and K % 16 == 0:
        if f == 1:
            need = (N * K // 2, N * K // 16)
            if _nbytes(src_q) < need[0] or (src_s is not None and _nbytes(src_s) < need[1]):
                raise ValueError(f"canonical NVFP4 planes too small: need {need[0]} + {need[1]} bytes")
        elif K % 32 == 0 and f in (2, 3, 4):
            need = N * (K // 32) * {2: 18, 3: 17, 4: 18}[f]
            if _nbytes(src_q) < need:
                raise ValueError(f"canonical blocks too small: need {need} bytes, got {_nbytes(src_q)}")
        if f in (1, 2, 3, 4) and (f == 1 or K % 32 == 0):
            _check_planes(f, N, K, dst_q, dst_s)
    with torch.cuda.device(dev):
        _check(lib().fp4_pack_layout(f, N, K, _ptr(src_q), _ptr(src_s), _ptr(dst_q), _ptr(dst_s), int(bool(validate)),
                                     _stream(stream)), "fp4_pack_layout")


def _product(name, fmt, M, N, K, q, s, global_scale, x, y, stream):
    if x.dtype != torch.bfloat16 or y.dtype != torch.float32:
        raise TypeError("x must be bfloat16 and y float32")
    if x.numel() < M * K or y.numel() < M * N:
        raise ValueError("x or y is smaller than M x K / M x N")
    f = _fmt(fmt)
    dev = _device(q, s, x, y)
    if M > 0 and N > 0 and K > 0:
        _check_planes(f, N, K, q, s)
    with torch.cuda.device(dev):
        _check(getattr(lib(), name)(f, M, N, K, _ptr(q), _ptr(s), float(global_scale), _ptr(x), _ptr(y),
                                    _stream(stream)), name)


def w4a16_gemv(fmt, M, N, K, q, s, global_scale, x, y, stream=None):
    _product("w4a16_gemv", fmt, M, N, K, q, s, global_scale, x, y, stream)


def w4a16_gemv_batched(fmt, M, items, stream=None):
    """items: sequence of (q, s, global_scale, x, y, N, K), one per matrix; all share fmt and M."""
    arr = (GemvItem * max(1, len(items)))()
    f = _fmt(fmt)
    tensors = []
    for i, (q, s, g, x, y, n, k) in enumerate(items):
        if x.dtype != torch.bfloat16 or y.dtype != torch.float32:
            raise TypeError("x must be bfloat16 and y float32")
        if x.numel() < M * k or y.numel() < M * n:
            raise ValueError("x or y is smaller than M x K / M x N")
        if M > 0 and n > 0 and k > 0:
            _check_planes(f, n, k, q, s)
        tensors += [q, s, x, y]
        arr[i] = GemvItem(_ptr(q), _ptr(s), _ptr(x), _ptr(y), n, k, float(g))
    with torch.cuda.device(_device(*tensors) if tensors else torch.cuda.current_device()):
        _check(lib().w4a16_gemv_batched(f, M, len(items), arr, _stream(stream)), "w4a16_gemv_batched")


def _workspace_bytes(name, fmt, M, N, K, device=None) -> int:
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        n = int(getattr(lib(), name)(_fmt(fmt), M, N, K))
    _check(n if n < 0 else 0, name)
    return n


def w4a16_gemm_workspace_bytes(fmt, M, N, K, device=None) -> int:
    """Workspace bytes w4a16_gemm_ws would use for this shape on `device` (default: the current one)."""
    return _workspace_bytes("w4a16_gemm_workspace_bytes", fmt, M, N, K, device)


def w4a16_matmul_workspace_bytes(fmt, M, N, K, device=None) -> int:
    """Workspace bytes w4a16_matmul_ws can use for this shape on `device` (0: it takes none)."""
    return _workspace_bytes("w4a16_matmul_workspace_bytes", fmt, M, N, K, device)


def _product_ws(name, fmt, M, N, K, q, s, global_scale, x, y, stream, workspace):
    """A product entry point that takes a workspace: `workspace` (a uint8 CUDA tensor) or, by default, one
    of the size the library asks for, allocated here from torch's caching allocator on the launch stream."""
    if x.dtype != torch.bfloat16 or y.dtype != torch.float32:
        raise TypeError("x must be bfloat16 and y float32")
    if x.numel() < M * K or y.numel() < M * N:
        raise ValueError("x or y is smaller than M x K / M x N")
    f = _fmt(fmt)
    dev = _device(q, s, x, y)
    if M > 0 and N > 0 and K > 0:
        _check_planes(f, N, K, q, s)
    with torch.cuda.device(dev):
        st = _stream(stream)
        if workspace is None and M > 0:
            query = "w4a16_gemm_workspace_bytes" if name == "w4a16_gemm_ws" else "w4a16_matmul_workspace_bytes"
            nbytes = _workspace_bytes(query, f, M, N, K, dev)
            if nbytes > 0:
                workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
                if stream is not None:
                    # the kernels run on `stream`, not necessarily the one the allocator recorded
                    ext = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(st)
                    workspace.record_stream(ext)
        ws_ptr, ws_bytes = (None, 0) if workspace is None else (_ptr(workspace), _nbytes(workspace))
        _check(getattr(lib(), name)(f, M, N, K, _ptr(q), _ptr(s), float(global_scale), _ptr(x), _ptr(y), ws_ptr,
                                    ws_bytes, st), name)


def w4a16_gemm(fmt, M, N, K, q, s, global_scale, x, y, stream=None, workspace=None):
    """The prefill product through w4a16_gemm_ws (K parts in a workspace where the launch rules split K)."""
    _product_ws("w4a16_gemm_ws", fmt, M, N, K, q, s, global_scale, x, y, stream, workspace)


def w4a16_gemm_noworkspace(fmt, M, N, K, q, s, global_scale, x, y, stream=None):
    """The C entry point w4a16_gemm itself (no workspace: at most the two-part atomic split)."""
    _product("w4a16_gemm", fmt, M, N, K, q, s, global_scale, x, y, stream)


def w4a16_gemm_noalloc(fmt, M, N, K, q, s, global_scale, x, y, stream=None):
    _product("w4a16_gemm_noalloc", fmt, M, N, K, q, s, global_scale, x, y, stream)


def w4a16_midm(fmt, M, N, K, q, s, global_scale, x, y, stream=None):
    _product("w4a16_midm", fmt, M, N, K, q, s, global_scale, x, y, stream)


def w4a16_matmul(fmt, M, N, K, q, s, global_scale, x, y, stream=None, workspace=None):
    """Dispatch on M through w4a16_matmul_ws (the prefill path with a workspace)."""
    _product_ws("w4a16_matmul_ws", fmt, M, N, K, q, s, global_scale, x, y, stream, workspace)


def fp4_dequant_f32(fmt, N, K, q, s, global_scale, w, stream=None):
    if w.dtype != torch.float32 or w.numel() < N * K:
        raise ValueError("w must be float32 with N x K elements")
    f = _fmt(fmt)
    dev = _device(q, s, w)
    if N > 0 and K > 0:
        _check_planes(f, N, K, q, s)
    with torch.cuda.device(dev):
        _check(lib().fp4_dequant_f32(f, N, K, _ptr(q), _ptr(s), float(global_scale), _ptr(w), _stream(stream)),
               "fp4_dequant_f32")


def fp4_quantize_nvfp4(N, K, w, wq, ws, g_out, stream=None):
    if w.dtype != torch.float32 or g_out.dtype != torch.float32:
        raise TypeError("w and g_out must be float32")
    if w.numel() < N * K or wq.numel() < N * K // 2 or ws.numel() < N * K // 16 or g_out.numel() < 1:
        raise ValueError("buffer too small")
    with torch.cuda.device(_device(w, wq, ws, g_out)):
        _check(lib().fp4_quantize_nvfp4(N, K, _ptr(w), _ptr(wq), _ptr(ws), _ptr(g_out), _stream(stream)),
               "fp4_quantize_nvfp4")


def fp4_quantize_rocmfp4(fmt, N, K, w, importance, blocks, stream=None):
    if w.dtype != torch.float32 or (importance is not None and importance.dtype != torch.float32):
        raise TypeError("w and importance must be float32")
    f = _fmt(fmt)
    bb = 18 if f == 2 else 17
    if w.numel() < N * K or blocks.numel() < N * (K // 32) * bb:
        raise ValueError("buffer too small")
    with torch.cuda.device(_device(w, importance, blocks)):
        _check(lib().fp4_quantize_rocmfp4(f, N, K, _ptr(w), _ptr(importance), _ptr(blocks), _stream(stream)),
               "fp4_quantize_rocmfp4")


def fp4_quantize_q4_0(N, K, w, blocks, stream=None):
    if w.dtype != torch.float32:
        raise TypeError("w must be float32")
    if w.numel() < N * K or blocks.numel() < N * (K // 32) * 18:
        raise ValueError("buffer too small")
    with torch.cuda.device(_device(w, blocks)):
        _check(lib().fp4_quantize_q4_0(N, K, _ptr(w), _ptr(blocks), _stream(stream)), "fp4_quantize_q4_0")


# ----------------------------------------------------------------------------------------------
# Convenience: a packed weight in kernel layout (allocation through torch, compute in the library)
# ----------------------------------------------------------------------------------------------

@dataclass
class PackedWeight:
    fmt: str
    N: int
    K: int
    q: torch.Tensor          # nibble plane (uint8)
    s: torch.Tensor          # scale plane (uint8)
    global_scale: float

    @staticmethod
    def empty(fmt: str, N: int, K: int, global_scale: float = 1.0, device="cuda") -> "PackedWeight":
        qb, sb = fp4_layout_bytes(fmt, N, K)
        return PackedWeight(fmt, N, K, torch.empty(qb, dtype=torch.uint8, device=device),
                            torch.empty(sb, dtype=torch.uint8, device=device), float(global_scale))

    @staticmethod
    def from_canonical(fmt: str, N: int, K: int, src_q: torch.Tensor, src_s: torch.Tensor | None,
                       global_scale: float = 1.0, stream=None, validate: bool = False) -> "PackedWeight":
        pw = PackedWeight.empty(fmt, N, K, global_scale, device=src_q.device)
        fp4_pack_layout(fmt, N, K, src_q, src_s, pw.q, pw.s, validate, stream)
        return pw

    @staticmethod
    def quantize(fmt: str, w: torch.Tensor, importance: torch.Tensor | None = None, stream=None) -> "PackedWeight":
        """Pack fp32 weights [N, K] on the GPU with the device packer, then repack to kernel layout."""
        N, K = w.shape
        w = w.contiguous()
        if fmt == "nvfp4":
            wq = torch.empty(N * K // 2, dtype=torch.uint8, device=w.device)
            ws = torch.empty(N * K // 16, dtype=torch.uint8, device=w.device)
            g = torch.empty(1, dtype=torch.float32, device=w.device)
            fp4_quantize_nvfp4(N, K, w, wq, ws, g, stream)
            gs = float(g.item())
            return PackedWeight.from_canonical(fmt, N, K, wq, ws, gs, stream=stream)
        blocks = torch.empty(N * (K // 32) * BLOCK_BYTES[fmt], dtype=torch.uint8, device=w.device)
        if fmt == "q4_0":
            if importance is not None:
                raise ValueError("the Q4_0 packer takes no importance")
            fp4_quantize_q4_0(N, K, w, blocks, stream)
        else:
            fp4_quantize_rocmfp4(fmt, N, K, w, importance, blocks, stream)
        return PackedWeight.from_canonical(fmt, N, K, blocks, None, 1.0, stream=stream)

    def matmul(self, x: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        M = x.shape[0]
        if x.shape[-1] != self.K:
            raise ValueError("x's last dimension must be K")
        if out is None:
            out = torch.empty(M, self.N, dtype=torch.float32, device=x.device)
        w4a16_matmul(self.fmt, M, self.N, self.K, self.q, self.s, self.global_scale, x.contiguous(), out, stream)
        return out

    def dequant(self, stream=None) -> torch.Tensor:
        w = torch.empty(self.N, self.K, dtype=torch.float32, device=self.q.device)
        fp4_dequant_f32(self.fmt, self.N, self.K, self.q, self.s, self.global_scale, w, stream)
        return w
