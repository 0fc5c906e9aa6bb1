"""GPU: fp4_pack_layout's scale validation (validate != 0) through the C ABI.

A NaN scale code (E4M3 / UE4M3 with the low 7 bits all ones; UE4M3's bit 7 is ignored, so 0xFF counts
too) or a non-finite Q4_0 FP16 scale must make the call return FP4_ERR_INVALID_SCALE before anything is
written; with validation off the same bytes repack and decode to NaN exactly as the oracle's FP32
dequantizer says. Both formats define their scales as finite (EdgeRock-4B-NVFP4 card, description;
ROCmFP4 design page, sections 02 and 03).
"""
import numpy as np
import pytest
import torch

from oracle import ref
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu

fp4 = pytest.importorskip("block_scaled_fp4_w4a16_amd")

INVALID_SCALE = -5


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _raw_pack(fmt, n, k, q, s, dq, ds, validate):
    f = fp4.FORMATS[fmt]
    return fp4.lib().fp4_pack_layout(f, n, k, q.data_ptr(), None if s is None else s.data_ptr(), dq.data_ptr(),
                                     ds.data_ptr(), validate, torch.cuda.current_stream().cuda_stream)


def _poison(fmt, packed, where, code):
    """A copy of the oracle-packed canonical bytes with scale number `where` replaced by `code`."""
    if fmt == "nvfp4":
        wq, ws, g = packed
        ws = ws.copy()
        ws.reshape(-1)[where] = code
        return (wq, ws, g)
    blocks, g = packed
    blocks = blocks.copy()
    flat = blocks.reshape(-1, blocks.shape[-1])
    if fmt == "rocmfp4_dual":
        flat[where // 2, where % 2] = code
    elif fmt == "rocmfp4_fast":
        flat[where, 0] = code
    else:                                   # q4_0: little-endian FP16
        flat[where, 0] = code & 0xFF
        flat[where, 1] = code >> 8
    return (blocks, g)


def _nscales(fmt, n, k):
    return n * k // 16 if fmt == "nvfp4" else n * (k // 32) * (2 if fmt == "rocmfp4_dual" else 1)


BAD = {"nvfp4": (0x7F, 0xFF), "rocmfp4_dual": (0x7F, 0xFF), "rocmfp4_fast": (0x7F, 0xFF),
       "q4_0": (0x7C00, 0xFC00, 0x7E00, 0xFFFF)}          # FP16 +inf, -inf, NaN, NaN


@pytest.mark.parametrize("fmt", gc.FMTS_ALL)
@pytest.mark.parametrize("n,k", [(16, 128), (37, 160)])
def test_invalid_scale_rejected_and_destination_untouched(fmt, n, k):
    print("CASE validate-reject", fmt, n, k, flush=True)
    _, packed = gc.make_case(fmt, n, k, cfg=71)
    qb, sb = fp4.fp4_layout_bytes(fmt, n, k)
    last = _nscales(fmt, n, k) - 1
    for where in (0, last // 2, last):
        for code in BAD[fmt]:
            bad = _poison(fmt, packed, where, code)
            q, s, _ = gc.canonical_tensors(fmt, bad)
            dq = torch.full((qb,), 0xA5, dtype=torch.uint8, device="cuda")
            ds = torch.full((sb,), 0x5A, dtype=torch.uint8, device="cuda")
            rc = _raw_pack(fmt, n, k, q, s, dq, ds, 1)
            torch.cuda.synchronize()
            assert rc == INVALID_SCALE, (fmt, where, hex(code), rc)
            assert bool((dq == 0xA5).all()) and bool((ds == 0x5A).all()), "destination written"
            with pytest.raises(RuntimeError, match="invalid scale"):
                fp4.fp4_pack_layout(fmt, n, k, q, s, dq, ds, validate=True)
    # a valid matrix right after a rejected one passes (the result word is cleared per call) and gives
    # the same planes as the unvalidated repack
    q, s, _ = gc.canonical_tensors(fmt, packed)
    dq1 = torch.empty(qb, dtype=torch.uint8, device="cuda")
    ds1 = torch.empty(sb, dtype=torch.uint8, device="cuda")
    dq0, ds0 = torch.empty_like(dq1), torch.empty_like(ds1)
    assert _raw_pack(fmt, n, k, q, s, dq1, ds1, 1) == 0
    assert _raw_pack(fmt, n, k, q, s, dq0, ds0, 0) == 0
    torch.cuda.synchronize()
    assert torch.equal(dq1, dq0) and torch.equal(ds1, ds0)


@pytest.mark.parametrize("fmt", gc.FMTS_ALL)
def test_largest_finite_scales_accepted(fmt):
    print("CASE validate-finite", fmt, flush=True)
    n, k = 32, 256
    _, packed = gc.make_case(fmt, n, k, cfg=72)
    codes = {"nvfp4": (0x7E, 0xFE), "rocmfp4_dual": (0x7E, 0xFE), "rocmfp4_fast": (0x7E, 0xFE),
             "q4_0": (0x7BFF, 0xFBFF)}[fmt]
    for code in codes:
        edge = _poison(fmt, packed, 3, code)
        q, s, _ = gc.canonical_tensors(fmt, edge)
        qb, sb = fp4.fp4_layout_bytes(fmt, n, k)
        dq = torch.empty(qb, dtype=torch.uint8, device="cuda")
        ds = torch.empty(sb, dtype=torch.uint8, device="cuda")
        assert _raw_pack(fmt, n, k, q, s, dq, ds, 1) == 0


@pytest.mark.parametrize("fmt", gc.FMTS_ALL)
def test_without_validation_nan_propagates_as_defined(fmt):
    print("CASE validate-off", fmt, flush=True)
    n, k = 37, 160
    _, packed = gc.make_case(fmt, n, k, cfg=73)
    bad = _poison(fmt, packed, 5, BAD[fmt][0])
    pw = gc.upload(fmt, n, k, bad)                  # validate off (the default)
    got = pw.dequant().cpu().numpy()
    want = ref.dequant_f32(fmt, bad)
    nonfinite = ~np.isfinite(want)
    assert nonfinite.any()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(np.isinf(got), np.isinf(want))
    assert np.array_equal(got[~nonfinite], want[~nonfinite])
