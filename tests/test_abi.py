"""The C-ABI library loads, exports every declared entry point and rejects bad arguments before
launching anything (runs without a GPU: every call here fails validation on the host)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4w4a16.h")

fp4 = pytest.importorskip("block_scaled_fp4_w4a16_amd")

OK, ARG, SHAPE, ALIGN, UNSUP, INVALID_SCALE, HIP = 0, -1, -2, -3, -4, -5, -6
FAKE = 1 << 20   # a 16-byte-aligned non-null address; never dereferenced by these calls
NVFP4, DUAL, FAST, Q4_0 = 1, 2, 3, 4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"fp4_pack_layout", "w4a16_gemv", "w4a16_gemm"} <= set(names)
    h = ctypes.CDLL(fp4.LIB_PATH)
    for n in names:
        assert hasattr(h, n), n


def test_version_and_status_strings():
    assert fp4.fp4_abi_version() == 3
    for st in (OK, ARG, SHAPE, ALIGN, UNSUP, INVALID_SCALE, HIP, 12345):
        assert isinstance(fp4.fp4_status_string(st), str) and fp4.fp4_status_string(st)
    # every status has its own text
    texts = [fp4.fp4_status_string(st) for st in (OK, ARG, SHAPE, ALIGN, UNSUP, INVALID_SCALE, HIP)]
    assert len(set(texts)) == len(texts)
    assert "scale" in fp4.fp4_status_string(INVALID_SCALE)
    assert fp4.fp4_status_string(12345) == "unknown status"


def test_header_declares_status_codes():
    text = open(HEADER).read()
    for name, value in (("FP4_OK", 0), ("FP4_ERR_ARG", -1), ("FP4_ERR_SHAPE", -2), ("FP4_ERR_ALIGN", -3),
                        ("FP4_ERR_UNSUPPORTED", -4), ("FP4_ERR_INVALID_SCALE", -5), ("FP4_ERR_HIP", -6)):
        assert re.search(rf"\b{name}\s*=\s*{value}\b", text), name
    assert re.search(r"FP4W4A16_ABI_VERSION\s+3\b", text)
    assert re.search(r"int fp4_pack_layout\([^)]*int validate, void\* stream\)", text)


def test_layout_bytes():
    # 16-row tiles x 128-wide chunks; 1 KiB of nibbles per unit; 8 (16-groups) or 4 (FAST) scale bytes per row
    assert fp4.fp4_layout_bytes("nvfp4", 2048, 2048) == (2048 * 2048 // 2, 2048 * 2048 // 16)
    assert fp4.fp4_layout_bytes("rocmfp4_dual", 4096, 4096) == (4096 * 4096 // 2, 4096 * 4096 // 16)
    assert fp4.fp4_layout_bytes("rocmfp4_fast", 14336, 4096) == (14336 * 4096 // 2, 14336 * 4096 // 32)
    assert fp4.fp4_layout_bytes("q4_0", 4096, 4096) == (4096 * 4096 // 2, 4096 * 4096 // 16)  # FP16 per 32
    # ragged: N = 17 -> 2 tiles, K = 160 -> 2 chunks
    assert fp4.fp4_layout_bytes("rocmfp4_dual", 17, 160) == (2 * 2 * 1024, 2 * 2 * 128)
    with pytest.raises(RuntimeError):
        fp4.fp4_layout_bytes("rocmfp4_fast", 16, 48)     # K not a multiple of 32
    with pytest.raises(RuntimeError):
        fp4.fp4_layout_bytes("nvfp4", 0, 64)


def test_layout_bytes_matches_weight_bytes_for_aligned_shapes():
    # the kernel layout stores exactly the canonical weight + scale bytes when N % 16 == K % 128 == 0
    from oracle import layouts
    for fmt in ("nvfp4", "rocmfp4_dual", "rocmfp4_fast", "q4_0"):
        q, s = fp4.fp4_layout_bytes(fmt, 256, 1024)
        assert q + s == layouts.canonical_bytes(fmt, 256, 1024)


def _raw():
    return fp4.lib()


@pytest.mark.parametrize("fn", ["w4a16_gemv", "w4a16_midm", "w4a16_gemm", "w4a16_matmul", "w4a16_gemm_noalloc"])
def test_product_argument_errors(fn):
    f = getattr(_raw(), fn)
    good = dict(fmt=NVFP4, M=1, N=16, K=64, q=FAKE, s=FAKE, g=1.0, x=FAKE, y=FAKE, st=None)

    def call(**kw):
        a = dict(good, **kw)
        return f(a["fmt"], a["M"], a["N"], a["K"], a["q"], a["s"], a["g"], a["x"], a["y"], a["st"])

    assert call(fmt=7) == ARG
    assert call(fmt=0) == ARG
    assert call(fmt=5) == ARG
    if fn in ("w4a16_midm", "w4a16_gemm", "w4a16_gemm_noalloc"):
        assert call(fmt=Q4_0) == UNSUP          # Q4_0 runs through the GEMV only
    else:
        assert call(fmt=Q4_0, K=48) == SHAPE   # Q4_0 needs K % 32 == 0
    assert call(q=None) == ARG
    assert call(s=None) == ARG
    assert call(x=None) == ARG
    assert call(y=None) == ARG
    assert call(K=40) == SHAPE                  # NVFP4 needs K % 16 == 0
    assert call(fmt=DUAL, K=48) == SHAPE        # ROCmFP4 needs K % 32 == 0
    assert call(N=0) == SHAPE
    assert call(K=0) == SHAPE
    assert call(M=-1) == SHAPE
    assert call(x=FAKE + 8) == ALIGN
    assert call(q=FAKE + 4) == ALIGN
    assert call(y=FAKE + 2) == ALIGN
    assert call(M=0, q=None, x=None) == OK     # M = 0 is a no-op
    assert call(N=1 << 31) == UNSUP
    if fn == "w4a16_gemv":
        assert call(M=17) == UNSUP
    if fn == "w4a16_midm":
        assert call(M=65) == UNSUP
    # K limits (32-bit buffer offsets): 2^24 for the GEMV and mid-M kernels, 2^22 for the GEMM
    if fn in ("w4a16_gemv", "w4a16_midm", "w4a16_matmul"):
        assert call(K=(1 << 24) + 16) == UNSUP
    else:
        assert call(M=128, K=(1 << 22) + 16) == UNSUP


@pytest.mark.parametrize("fn", ["w4a16_gemm_ws", "w4a16_matmul_ws"])
def test_workspace_product_argument_errors(fn):
    f = getattr(_raw(), fn)
    M = 128  # the prefill path (w4a16_matmul_ws dispatches to it above M = 64)

    def call(fmt=NVFP4, K=64, x=FAKE, ws=FAKE, wsb=1 << 20):
        return f(fmt, M, 16, K, FAKE, FAKE, 1.0, x, FAKE, ws, wsb, None)

    assert call(fmt=7) == ARG
    assert call(K=40) == SHAPE
    assert call(x=FAKE + 8) == ALIGN
    assert call(ws=FAKE + 4) == ALIGN          # the workspace must be 16-byte aligned
    assert call(fmt=Q4_0) == UNSUP
    assert f(NVFP4, 0, 16, 64, None, None, 1.0, None, None, None, 0, None) == OK


def test_workspace_bytes_query():
    r = _raw()
    q = r.w4a16_gemm_workspace_bytes
    assert q(7, 128, 2560, 9728) == ARG
    assert q(Q4_0, 128, 2560, 9728) == UNSUP
    assert q(NVFP4, 128, 2560, 40) == SHAPE
    assert q(NVFP4, -1, 2560, 9728) == SHAPE
    assert q(NVFP4, 0, 2560, 9728) == 0
    cus = 256  # without a GPU the library plans for a 256-CU device
    # the prefill shape fills the device: no K parts
    assert q(NVFP4, 2048, 14336, 4096) == 0
    # a 2560 x 9728 projection at M = 128 has 20 tiles of 128 x 128: the split rule takes 9 K parts (180 CUs)
    assert q(NVFP4, 128, 2560, 9728) == 9 * 128 * 2560 * 4
    # the parts' planes never exceed 64 KiB per CU (one round of 128 x 128 tiles), so the 16 MiB static
    # scratch of the no-allocation entry point covers every split on a 256-CU device
    worst = 0
    for m in (65, 96, 128, 160, 192, 256, 300, 512):
        for n in (128, 1000, 2560, 4096, 9728, 14336):
            for k in (128, 1024, 2560, 4096, 9728):
                b = q(DUAL, m, n, k)
                assert b >= 0 and b % (4 * m * n) == 0
                worst = max(worst, b)
    assert 0 < worst <= cus * 64 * 1024


def test_matmul_workspace_bytes_query():
    r = _raw()
    qm, qg = r.w4a16_matmul_workspace_bytes, r.w4a16_gemm_workspace_bytes
    assert qm(7, 56, 2560, 9728) == ARG
    assert qm(NVFP4, 56, 2560, 40) == SHAPE
    assert qm(NVFP4, 8, 2560, 9728) == 0              # the GEMV takes no workspace
    assert qm(NVFP4, 47, 2560, 9728) == 0             # nor the mid-M kernel
    assert qm(Q4_0, 56, 2560, 9728) == 0
    assert qm(NVFP4, 56, 4096, 4096) == 0             # 16 M weights: the mid-M kernel
    for m in (48, 56, 64, 128):                       # the GEMM's K parts
        assert qm(NVFP4, m, 2560, 9728) == qg(NVFP4, m, 2560, 9728) > 0
    assert qm(Q4_0, 128, 2560, 9728) == UNSUP


@pytest.mark.parametrize("validate", [0, 1])
def test_pack_layout_argument_errors(validate):
    # argument checks come before the validation pass, so these fail on the host with or without it
    f = _raw().fp4_pack_layout
    v = validate
    assert f(Q4_0, 16, 64, FAKE, FAKE, FAKE, FAKE, v, None) == ARG       # Q4_0 carries scales in blocks
    assert f(NVFP4, 16, 64, FAKE, None, FAKE, FAKE, v, None) == ARG      # NVFP4 needs the scale plane
    assert f(DUAL, 16, 64, FAKE, FAKE, FAKE, FAKE, v, None) == ARG       # ROCmFP4 carries scales in blocks
    assert f(FAST, 16, 48, FAKE, None, FAKE, FAKE, v, None) == SHAPE
    assert f(FAST, 16, 64, FAKE, None, FAKE + 4, FAKE, v, None) == ALIGN
    assert f(9, 16, 64, FAKE, None, FAKE, FAKE, v, None) == ARG
    assert f(DUAL, 16, 64, None, None, FAKE, FAKE, v, None) == ARG
    assert f(DUAL, 0, 64, FAKE, None, FAKE, FAKE, v, None) == SHAPE


def test_dequant_and_quantize_argument_errors():
    r = _raw()
    assert r.fp4_dequant_f32(NVFP4, 16, 40, FAKE, FAKE, 1.0, FAKE, None) == SHAPE
    assert r.fp4_dequant_f32(NVFP4, 16, 64, None, FAKE, 1.0, FAKE, None) == ARG
    assert r.fp4_quantize_nvfp4(16, 40, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
    assert r.fp4_quantize_nvfp4(16, 64, None, FAKE, FAKE, FAKE, None) == ARG
    assert r.fp4_quantize_rocmfp4(NVFP4, 16, 64, FAKE, None, FAKE, None) == ARG
    assert r.fp4_quantize_rocmfp4(DUAL, 16, 48, FAKE, None, FAKE, None) == SHAPE
    assert r.fp4_quantize_rocmfp4(FAST, 16, 64, FAKE + 4, None, FAKE, None) == ALIGN
    assert r.fp4_quantize_rocmfp4(Q4_0, 16, 64, FAKE, None, FAKE, None) == ARG
    assert r.fp4_quantize_q4_0(16, 48, FAKE, FAKE, None) == SHAPE
    assert r.fp4_quantize_q4_0(16, 64, None, FAKE, None) == ARG
    assert r.fp4_quantize_q4_0(16, 64, FAKE + 4, FAKE, None) == ALIGN
    assert r.fp4_dequant_f32(Q4_0, 16, 48, FAKE, FAKE, 1.0, FAKE, None) == SHAPE


def test_python_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        fp4._ptr(torch.zeros(4))


def test_gemv_batched_argument_errors():
    f = _raw().w4a16_gemv_batched
    Item = fp4.GemvItem

    def items(*specs):
        arr = (Item * max(1, len(specs)))()
        for i, kw in enumerate(specs):
            a = dict(q=FAKE, s=FAKE, x_bf16=FAKE, y=FAKE, N=16, K=64, global_scale=1.0)
            a.update(kw)
            arr[i] = Item(a["q"], a["s"], a["x_bf16"], a["y"], a["N"], a["K"], a["global_scale"])
        return arr

    good = {}
    assert f(7, 1, 1, items(good), None) == ARG
    assert f(NVFP4, 17, 1, items(good), None) == UNSUP
    assert f(NVFP4, -1, 1, items(good), None) == SHAPE
    assert f(NVFP4, 1, -1, items(good), None) == ARG
    assert f(NVFP4, 1, fp4.GEMV_MAX_ITEMS + 1, items(good), None) == UNSUP
    assert f(NVFP4, 1, 1, None, None) == ARG
    assert f(NVFP4, 1, 0, None, None) == OK                    # no items: no-op
    assert f(NVFP4, 0, 2, items(good, dict(q=None)), None) == OK   # M = 0: no-op
    # the first failing item decides the status
    assert f(NVFP4, 1, 3, items(good, dict(K=40), dict(q=None)), None) == SHAPE
    assert f(NVFP4, 1, 2, items(good, dict(y=FAKE + 2)), None) == ALIGN
    assert f(DUAL, 1, 2, items(good, dict(K=48)), None) == SHAPE
    assert f(NVFP4, 1, 2, items(good, dict(x_bf16=None)), None) == ARG
    assert f(NVFP4, 1, 1, items(dict(K=1 << 25)), None) == UNSUP
