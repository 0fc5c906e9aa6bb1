"""GPU parity of the HIP path against the CPU oracle (MI355X; every call goes through the C ABI).

Bars: dequantized weights bit-exact in FP32 (+0 == -0); products within
|y - y_ref| <= 2e-3 * sum|x w| + 1e-6 elementwise; packers byte-exact.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import layouts, pack, ref
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu

fp4 = pytest.importorskip("block_scaled_fp4_w4a16_amd")


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _announce(*a):
    print("CASE", *a, flush=True)


# ------------------------------------------------------------------ dequant (bit-exact)

@pytest.mark.parametrize("fmt", gc.FMTS_ALL)
@pytest.mark.parametrize("n,k", [(16, 128), (37, 160), (64, 1024), (5, 32 * 7)])
def test_dequant_bit_exact(fmt, n, k):
    if fmt == "nvfp4" and k % 16:
        pytest.skip()
    _announce("dequant", fmt, n, k)
    w, packed = gc.make_case(fmt, n, k, cfg=51)
    pw = gc.upload(fmt, n, k, packed)
    got = pw.dequant().cpu().numpy()
    want = ref.dequant_f32(fmt, packed)
    assert got.shape == want.shape
    assert np.array_equal(got, want)  # == treats +0 and -0 as equal


@pytest.mark.parametrize("fmt", gc.FMTS_ALL)
def test_dequant_all_codes_and_scales(fmt):
    # every nibble code against every finite scale byte (and NaN scales for NVFP4)
    _announce("dequant-all-codes", fmt)
    rng = np.random.default_rng(8)
    n, k = 128, 512
    if fmt == "nvfp4":
        wq = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
        ws = (np.arange(n * k // 16) % 256).astype(np.uint8).reshape(n, k // 16)
        packed = (wq, ws, np.float32(0.37))
    elif fmt == "q4_0":
        blocks = rng.integers(0, 256, size=(n, k // 32, 18), dtype=np.uint8)
        d = np.arange(n * (k // 32), dtype=np.uint32) * 7 % (1 << 16)
        d = d[((d >> 10) & 31) != 31][: n * (k // 32)]         # finite FP16 scales of both signs
        d = np.resize(d, n * (k // 32)).astype(np.uint16).reshape(n, k // 32)
        blocks[:, :, 0] = d & 0xFF
        blocks[:, :, 1] = d >> 8
        packed = (blocks, np.float32(1.0))
    else:
        bb = layouts.BLOCK_BYTES[fmt]
        blocks = rng.integers(0, 256, size=(n, k // 32, bb), dtype=np.uint8)
        ns = layouts.SCALES_PER_BLOCK[fmt]
        blocks[:, :, :ns] = (np.arange(n * (k // 32) * ns) % 127).astype(np.uint8).reshape(n, k // 32, ns)
        packed = (blocks, np.float32(1.0))
    pw = gc.upload(fmt, n, k, packed)
    got = pw.dequant().cpu().numpy()
    want = ref.dequant_f32(fmt, packed)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


# ------------------------------------------------------------------ GEMV (M <= 16)

@pytest.mark.parametrize("fmt", gc.FMTS_ALL)
@pytest.mark.parametrize("m", list(range(1, 17)))
def test_gemv_small_shapes(fmt, m):
    # at M = 1: (48, 256), (37, 160), (256, 1536) and (24, 4096) fill every chunk slot of every wave;
    # (40, 2560) leaves the last slot of half the waves past the last chunk; (20, 96) is one partial chunk
    # on the two-slot kernel
    for (n, k) in [(48, 256), (37, 160), (256, 1536), (24, 4096), (40, 2560), (20, 96)]:
        _announce("gemv", fmt, m, n, k)
        w, packed = gc.make_case(fmt, n, k, cfg=52, mat=n)
        pw = gc.upload(fmt, n, k, packed)
        x_bits = synth.activations(m, k, cfg=52, mat=k)
        y = torch.full((m, n), float("nan"), device="cuda")
        fp4.w4a16_gemv(fmt, m, n, k, pw.q, pw.s, pw.global_scale, gc.x_tensor(x_bits), y)
        torch.cuda.synchronize()
        gc.check_product(fmt, packed, x_bits, y, label=f"gemv {fmt} M={m} {n}x{k}")


@pytest.mark.parametrize("fmt", gc.FMTS_ALL)
@pytest.mark.parametrize("m", [1, 2, 4])
def test_gemv_long_k_batches(fmt, m):
    # K = 8288: 65 chunks, the last partial: 5 chunk slots per wave at 16 waves, all in one batch.
    # K = 14464: 113 chunks, more than 6 slots per wave, so each wave runs several batches of chunk slots
    # with the next batch prefetched. The ring kernel is not picked at this grid size.
    for n, k in [(40, 8288), (24, 14464)]:
        _announce("gemv-long-k", fmt, m, n, k)
        w, packed = gc.make_case(fmt, n, k, cfg=64, mat=m)
        pw = gc.upload(fmt, n, k, packed)
        x_bits = synth.activations(m, k, cfg=64, mat=k + m)
        y = torch.full((m, n), float("nan"), device="cuda")
        fp4.w4a16_gemv(fmt, m, n, k, pw.q, pw.s, pw.global_scale, gc.x_tensor(x_bits), y)
        torch.cuda.synchronize()
        gc.check_product(fmt, packed, x_bits, y, label=f"gemv-long-k {fmt} M={m} K={k}")


@pytest.mark.parametrize("fmt", ["nvfp4", "rocmfp4_fast", "q4_0"])
def test_very_long_k(fmt):
    # K = 2^20 + 32 (8193 chunks, the last partial) through a single 16-row tile: the GEMV's batch loop
    # and the mid-M chain then run hundreds of steps per wave, and the x and plane offsets reach 2^21.
    n, k = 16, (1 << 20) + 32
    w, packed = gc.make_case(fmt, n, k, cfg=65, mat=0)
    pw = gc.upload(fmt, n, k, packed)
    for m in (1, 2, 9, 16):
        _announce("gemv-very-long-k", fmt, m, n, k)
        x_bits = synth.activations(m, k, cfg=65, mat=m)
        y = torch.full((m, n), float("nan"), device="cuda")
        fp4.w4a16_gemv(fmt, m, n, k, pw.q, pw.s, pw.global_scale, gc.x_tensor(x_bits), y)
        torch.cuda.synchronize()
        gc.check_product(fmt, packed, x_bits, y, label=f"gemv-very-long-k {fmt} M={m}")
    if fmt == "q4_0":
        return  # the matrix-core paths do not take Q4_0
    m = 33
    _announce("midm-very-long-k", fmt, m, n, k)
    x_bits = synth.activations(m, k, cfg=65, mat=m)
    y = torch.full((m, n), float("nan"), device="cuda")
    fp4.w4a16_midm(fmt, m, n, k, pw.q, pw.s, pw.global_scale, gc.x_tensor(x_bits), y)
    torch.cuda.synchronize()
    gc.check_product(fmt, packed, x_bits, y, label=f"midm-very-long-k {fmt} M={m}")


@pytest.mark.parametrize("fmt", ["nvfp4", "rocmfp4_fast"])
def test_gemm_very_long_k(fmt):
    # K = 2^20 + 32 on a one-tile grid (N = 32 of a 256-column tile, M = 65 of a 256-row one): 16385
    # stages through the ring, with the small-grid K split.
    m, n, k = 65, 32, (1 << 20) + 32
    _announce("gemm-very-long-k", fmt, m, n, k)
    w, packed = gc.make_case(fmt, n, k, cfg=66, mat=0)
    pw = gc.upload(fmt, n, k, packed)
    x_bits = synth.activations(m, k, cfg=66, mat=m)
    y = torch.full((m, n), float("nan"), device="cuda")
    fp4.w4a16_gemm(fmt, m, n, k, pw.q, pw.s, pw.global_scale, gc.x_tensor(x_bits), y)
    torch.cuda.synchronize()
    gc.check_product(fmt, packed, x_bits, y, label=f"gemm-very-long-k {fmt}")


def test_gemv_ring_forced(tmp_path):
    # The long-K ring kernel (M = 1), switched on for small grids (FP4_GEMV_RING=1, in a child process: the
    # library reads its tuning overrides once per process): a ragged last tile, a partial last 128-wide chunk,
    # chunk counts that are not a multiple of 16 waves x 3 slots, waves with no chunk at all (10 chunks for
    # 16 waves), and the largest K it takes (256 chunks, 64 KiB of staged x).
    cases = {}
    for fmt in gc.FMTS_ALL:
        for n, k in [(200, 8288), (37, 1184), (16, 32768)]:
            _announce("gemv-ring", fmt, n, k)
            w, packed = gc.make_case(fmt, n, k, cfg=59, mat=n)
            pw = gc.upload(fmt, n, k, packed)
            x_bits = synth.activations(1, k, cfg=59, mat=k)
            name = f"{fmt}_{n}_{k}"
            gc.save_case(tmp_path, name, "gemv", fmt, 1, n, k, pw, x_bits)
            cases[name] = (fmt, packed, x_bits)
    ys = gc.run_variant(tmp_path, {"FP4_GEMV_RING": "1"})
    for name, (fmt, packed, x_bits) in cases.items():
        gc.check_product(fmt, packed, x_bits, torch.from_numpy(ys[name]), label=f"gemv-ring {name}")


def test_gemv_slot_override(tmp_path):
    # FP4_GEMV_U=4 (child process) gives M = 1 more chunk slots per wave than the shape needs: with 20
    # chunks (8 waves x 4 slots) slots before the last lie past the last chunk, so every slot is tested;
    # with 12 chunks (4 waves x 4 slots) only the last slot of every wave is empty. Results must not change.
    cases = {}
    for fmt in gc.FMTS_ALL:
        for (n, k) in [(40, 2560), (256, 1536)]:
            _announce("gemv-slot-override", fmt, n, k)
            w, packed = gc.make_case(fmt, n, k, cfg=53, mat=n)
            pw = gc.upload(fmt, n, k, packed)
            x_bits = synth.activations(1, k, cfg=53, mat=k)
            name = f"{fmt}_{n}_{k}"
            gc.save_case(tmp_path, name, "gemv", fmt, 1, n, k, pw, x_bits)
            cases[name] = (fmt, packed, x_bits)
    ys = gc.run_variant(tmp_path, {"FP4_GEMV_U": "4"})
    for name, (fmt, packed, x_bits) in cases.items():
        gc.check_product(fmt, packed, x_bits, torch.from_numpy(ys[name]), label=f"gemv-slot-override {name}")


def test_gemv_one_batch_off(tmp_path):
    # With FP4_ONE_BATCH=0 (child process) 2 <= M <= 8 takes the batch loop (M <= 4) or the mid-M kernel
    # instead of the one-batch GEMV: the paths that the shape rules still pick where one batch does not
    # fit, on the shapes of the default-path test above
    cases = {}
    for fmt in gc.FMTS_ALL:
        for m in (2, 3, 4, 5, 8):
            for (n, k) in [(37, 160), (256, 1536)]:
                _announce("gemv-one-batch-off", fmt, m, n, k)
                w, packed = gc.make_case(fmt, n, k, cfg=52, mat=n)
                pw = gc.upload(fmt, n, k, packed)
                x_bits = synth.activations(m, k, cfg=52, mat=k)
                name = f"{fmt}_{m}_{n}_{k}"
                gc.save_case(tmp_path, name, "gemv", fmt, m, n, k, pw, x_bits)
                cases[name] = (fmt, packed, x_bits)
    ys = gc.run_variant(tmp_path, {"FP4_ONE_BATCH": "0"})
    for name, (fmt, packed, x_bits) in cases.items():
        gc.check_product(fmt, packed, x_bits, torch.from_numpy(ys[name]), label=f"gemv-one-batch-off {name}")


def test_gemv_ring_full_grid():
    # a grid of 512 tiles with 65 chunks per row: the shape rule itself picks the ring kernel on a
    # 256-CU GPU; sampled rows are checked
    fmt, n, k = "nvfp4", 8192, 8320
    _announce("gemv-ring-grid", fmt, n, k)
    w, packed = gc.make_case(fmt, n, k, cfg=58)
    del w
    pw = gc.upload(fmt, n, k, packed)
    x_bits = synth.activations(1, k, cfg=58, mat=1)
    y = torch.full((1, n), float("nan"), device="cuda")
    fp4.w4a16_gemv(fmt, 1, n, k, pw.q, pw.s, pw.global_scale, gc.x_tensor(x_bits), y)
    torch.cuda.synchronize()
    assert not torch.isnan(y).any()
    rng = np.random.default_rng(58)
    cols = np.unique(np.concatenate([[0, 15, 16, n - 17, n - 1], rng.choice(n, 91, replace=False)]))
    gc.check_product(fmt, packed, x_bits, y, cols=cols, label=f"gemv-ring-grid {n}x{k}")


@pytest.mark.parametrize("fmt", gc.FMTS_ALL)
def test_gemv_one_hot_returns_weight_columns_exactly(fmt):
    # x = e_k gives y[:, n] = W32[n, k] exactly (a single product, times g)
    n, k = 64, 256
    _announce("gemv-one-hot", fmt)
    w, packed = gc.make_case(fmt, n, k, cfg=53)
    pw = gc.upload(fmt, n, k, packed)
    ks = np.arange(0, k, 17)[:16]
    x_bits = np.zeros((len(ks), k), np.uint16)
    x_bits[np.arange(len(ks)), ks] = 0x3F80
    y = torch.empty((len(ks), n), device="cuda")
    fp4.w4a16_gemv(fmt, len(ks), n, k, pw.q, pw.s, pw.global_scale, gc.x_tensor(x_bits), y)
    torch.cuda.synchronize()
    want = ref.dequant_f32(fmt, packed)[:, ks].T
    assert np.array_equal(y.cpu().numpy(), want)


def test_gemv_canary_and_determinism():
    fmt, m, n, k = "rocmfp4_dual", 3, 40, 512
    _announce("gemv-canary", fmt)
    w, packed = gc.make_case(fmt, n, k, cfg=54)
    pw = gc.upload(fmt, n, k, packed)
    x = gc.x_tensor(synth.activations(m, k, cfg=54))
    buf = torch.full((m * n + 64,), 12345.0, device="cuda")
    y1 = buf[32:32 + m * n]
    fp4.w4a16_gemv(fmt, m, n, k, pw.q, pw.s, 1.0, x, y1)
    torch.cuda.synchronize()
    first = y1.clone()
    for _ in range(3):
        fp4.w4a16_gemv(fmt, m, n, k, pw.q, pw.s, 1.0, x, y1)
    torch.cuda.synchronize()
    assert torch.equal(first, y1)                         # bitwise repeatable
    assert torch.all(buf[:32] == 12345.0) and torch.all(buf[32 + m * n:] == 12345.0)


def test_products_on_side_streams():
    # The library keeps no per-call state: the GEMV, mid-M kernel and GEMM launched on two side streams at
    # once, each call with its own output, give the bytes they give on the current stream one at a time.
    fmt, n, k = "rocmfp4_dual", 400, 1024
    _announce("side-streams", fmt)
    cases = []
    for mat, m in enumerate((1, 9, 96)):
        w, packed = gc.make_case(fmt, n, k, cfg=66, mat=mat)
        pw = gc.upload(fmt, n, k, packed)
        x_bits = synth.activations(m, k, cfg=66, mat=mat)
        x = gc.x_tensor(x_bits)
        ref_y = torch.full((m, n), float("nan"), device="cuda")
        fp4.w4a16_matmul(fmt, m, n, k, pw.q, pw.s, pw.global_scale, x, ref_y)
        torch.cuda.synchronize()
        gc.check_product(fmt, packed, x_bits, ref_y, label=f"side-streams M={m}")
        cases.append((m, pw, x, ref_y))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.full((m, n), float("nan"), device="cuda") for (m, _, _, _) in cases for _ in streams]
    for rep in range(3):
        i = 0
        for (m, pw, x, _) in cases:
            for st in streams:
                st.wait_stream(torch.cuda.current_stream())
                fp4.w4a16_matmul(fmt, m, n, k, pw.q, pw.s, pw.global_scale, x, outs[i], stream=st)
                i += 1
    torch.cuda.synchronize()
    i = 0
    for (m, pw, x, ref_y) in cases:
        for st in streams:
            assert torch.equal(outs[i], ref_y), f"M={m}: side-stream result differs"
            i += 1


def test_binding_rejects_short_planes_and_mixed_devices():
    # The binding checks buffer sizes the C ABI cannot see (raw pointers) before anything is launched.
    fmt, n, k = "rocmfp4_dual", 64, 256
    w, packed = gc.make_case(fmt, n, k, cfg=68)
    pw = gc.upload(fmt, n, k, packed)
    x = torch.zeros((1, k), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((1, n), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        fp4.w4a16_matmul(fmt, 1, n, k, pw.q[:-16], pw.s, 1.0, x, y)
    with pytest.raises(ValueError):
        fp4.w4a16_matmul(fmt, 1, n, k, pw.q, pw.s[:-1], 1.0, x, y)
    with pytest.raises(ValueError):
        fp4.w4a16_matmul(fmt, 1, n, k, pw.q, pw.s, 1.0, x.cpu(), y)
    with pytest.raises(ValueError):
        fp4.fp4_dequant_f32(fmt, n, k, pw.q[:100], pw.s, 1.0, torch.empty(n * k, device="cuda"))
    blocks = torch.zeros(n * (k // 32) * 18, dtype=torch.uint8, device="cuda")
    dq, ds = torch.empty_like(pw.q), torch.empty_like(pw.s)
    with pytest.raises(ValueError):
        fp4.fp4_pack_layout(fmt, n, k, blocks[:-1], None, dq, ds)
    with pytest.raises(ValueError):
        fp4.fp4_pack_layout(fmt, n, k, blocks, None, dq[:-1], ds)
    fp4.fp4_pack_layout(fmt, n, k, blocks, None, dq, ds)   # the full-size call still goes through
    torch.cuda.synchronize()


def test_gemv_m0_is_noop():
    y = torch.full((4,), 7.0, device="cuda")
    q = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    fp4.w4a16_gemv("nvfp4", 0, 16, 128, q, q, 1.0, torch.zeros(128, dtype=torch.bfloat16, device="cuda"), y)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


# ------------------------------------------------------------------ batched GEMV

@pytest.mark.parametrize("fmt", gc.FMTS_ALL)
@pytest.mark.parametrize("m", list(range(1, 17)))
def test_gemv_batched_matches_oracle(fmt, m):
    # matrices of different N and K (ragged tiles and chunks), two of them sharing one x, with
    # canaries around every y
    shapes = [(48, 256), (37, 160), (256, 1536), (16, 32 if fmt != "nvfp4" else 16), (130, 256)]
    _announce("gemv-batched", fmt, m, shapes)
    cases, items, bufs = [], [], []
    shared_x = None
    for i, (n, k) in enumerate(shapes):
        w, packed = gc.make_case(fmt, n, k, cfg=58, mat=100 * i + n)
        pw = gc.upload(fmt, n, k, packed)
        if i == 4:                      # same K as item 0: reuse its x
            x_bits = cases[0][2]
            x = shared_x
        else:
            x_bits = synth.activations(m, k, cfg=58, mat=1000 * i + k)
            x = gc.x_tensor(x_bits)
        if i == 0:
            shared_x = x
        buf = torch.full((m * n + 64,), 12345.0, device="cuda")
        y = buf[32:32 + m * n]
        cases.append((packed, pw, x_bits, y, buf, n, k))
        items.append((pw.q, pw.s, pw.global_scale, x, y, n, k))
    fp4.w4a16_gemv_batched(fmt, m, items)
    torch.cuda.synchronize()
    for (packed, pw, x_bits, y, buf, n, k) in cases:
        gc.check_product(fmt, packed, x_bits, y.view(m, n), label=f"batched {fmt} M={m} {n}x{k}")
        assert torch.all(buf[:32] == 12345.0) and torch.all(buf[32 + m * n:] == 12345.0)


@pytest.mark.parametrize("fmt", gc.FMTS_ALL)
@pytest.mark.parametrize("count", [3, 5])
def test_gemv_batched_equal_k(fmt, count):
    # grouped M = 1 launches whose matrices all have K = 1536 (12 chunks: 4 waves of 3 slots, every slot
    # holding a chunk, the straight-line form), with ragged N and one shared x; 3 matrices take the
    # 4-entry item table, 5 the 32-entry one
    m, k = 1, 1536
    shapes = [(40, k), (24, k), (130, k), (16, k), (77, k)][:count]
    _announce("gemv-batched-equal-k", fmt, count)
    x_bits = synth.activations(m, k, cfg=62, mat=count)
    x = gc.x_tensor(x_bits)
    items, cases = [], []
    for i, (n, kk) in enumerate(shapes):
        w, packed = gc.make_case(fmt, n, kk, cfg=62, mat=10 * count + i)
        pw = gc.upload(fmt, n, kk, packed)
        y = torch.full((m, n), float("nan"), device="cuda")
        items.append((pw.q, pw.s, pw.global_scale, x, y, n, kk))
        cases.append((packed, y, n))
    fp4.w4a16_gemv_batched(fmt, m, items)
    torch.cuda.synchronize()
    for packed, y, n in cases:
        gc.check_product(fmt, packed, x_bits, y, label=f"batched-equal-k {fmt} {count} {n}x{k}")


@pytest.mark.parametrize("count", [1, 2, 3, 4])
def test_gemv_batched_small_counts(count):
    # launches of up to four matrices pass a smaller item table; each output against the oracle, and a
    # single item bitwise equal to the single-matrix entry point (same kernel and wave count)
    fmt, m = "rocmfp4_dual", 1
    shapes = [(80, 384), (37, 160), (256, 4096), (16, 32)][:count]
    _announce("gemv-batched-small", fmt, m, shapes)
    items, cases = [], []
    for i, (n, k) in enumerate(shapes):
        w, packed = gc.make_case(fmt, n, k, cfg=61, mat=i)
        pw = gc.upload(fmt, n, k, packed)
        x_bits = synth.activations(m, k, cfg=61, mat=i)
        x = gc.x_tensor(x_bits)
        y = torch.full((m, n), float("nan"), device="cuda")
        items.append((pw.q, pw.s, pw.global_scale, x, y, n, k))
        cases.append((packed, pw, x, x_bits, y, n, k))
    fp4.w4a16_gemv_batched(fmt, m, items)
    torch.cuda.synchronize()
    for packed, pw, x, x_bits, y, n, k in cases:
        gc.check_product(fmt, packed, x_bits, y, label=f"batched-small {count} {n}x{k}")
    if count == 1:
        packed, pw, x, x_bits, y, n, k = cases[0]
        y1 = torch.empty_like(y)
        fp4.w4a16_gemv(fmt, m, n, k, pw.q, pw.s, pw.global_scale, x, y1)
        torch.cuda.synchronize()
        assert torch.equal(y1, y)


@pytest.mark.parametrize("m", [1, 3, 6])
@pytest.mark.parametrize("longest_k", [9728, 14464])
def test_gemv_batched_long_k(m, longest_k):
    # two matrices of K = 9728 (76 chunks: 5 chunk slots per wave at 16 waves, the one-batch form at
    # M <= 4) and, in the second case, one of K = 14464 (113 chunks: more slots than one batch holds,
    # so the whole group takes the prefetching batch loop); M = 6 takes the grouped mid-M kernel
    fmt = "rocmfp4_dual"
    shapes = [(48, 9728), (37, 9728)] + ([(16, 14464)] if longest_k > 9728 else [])
    _announce("gemv-batched-long-k", fmt, m, shapes)
    items, cases = [], []
    for i, (n, k) in enumerate(shapes):
        w, packed = gc.make_case(fmt, n, k, cfg=62, mat=i)
        pw = gc.upload(fmt, n, k, packed)
        x_bits = synth.activations(m, k, cfg=62, mat=i)
        y = torch.full((m, n), float("nan"), device="cuda")
        items.append((pw.q, pw.s, pw.global_scale, gc.x_tensor(x_bits), y, n, k))
        cases.append((packed, x_bits, y, n, k))
    fp4.w4a16_gemv_batched(fmt, m, items)
    torch.cuda.synchronize()
    for packed, x_bits, y, n, k in cases:
        gc.check_product(fmt, packed, x_bits, y, label=f"batched-long-k M={m} {n}x{k}")


@pytest.mark.parametrize("fmt,m", [("nvfp4", 2), ("rocmfp4_fast", 9), ("q4_0", 16)])
def test_gemv_batched_many_items_and_repeatability(fmt, m):
    # the full item count; every item a different matrix; outputs bitwise repeatable (M = 2: the GEMV's
    # one-batch form; 9 and 16: the grouped mid-M kernel)
    _announce("gemv-batched-max", fmt, m)
    items, cases = [], []
    for i in range(fp4.GEMV_MAX_ITEMS):
        n, k = 16 * (1 + i % 5), 128 * (1 + i % 3)
        w, packed = gc.make_case(fmt, n, k, cfg=59, mat=i)
        pw = gc.upload(fmt, n, k, packed)
        x_bits = synth.activations(m, k, cfg=59, mat=i)
        y = torch.full((m, n), float("nan"), device="cuda")
        items.append((pw.q, pw.s, pw.global_scale, gc.x_tensor(x_bits), y, n, k))
        cases.append((packed, x_bits, y))
    fp4.w4a16_gemv_batched(fmt, m, items)
    torch.cuda.synchronize()
    first = [c[2].clone() for c in cases]
    for packed, x_bits, y in cases:
        gc.check_product(fmt, packed, x_bits, y, label="batched-max")
    fp4.w4a16_gemv_batched(fmt, m, items)
    torch.cuda.synchronize()
    for f, (_, _, y) in zip(first, cases):
        assert torch.equal(f, y)


# ------------------------------------------------------------------ mid-M

@pytest.mark.parametrize("fmt", gc.FMTS)
@pytest.mark.parametrize("m", list(range(1, 65)))
def test_midm_shapes(fmt, m):
    for (n, k) in [(48, 256), (37, 160), (256, 1536)]:
        _announce("midm", fmt, m, n, k)
        w, packed = gc.make_case(fmt, n, k, cfg=60, mat=n)
        pw = gc.upload(fmt, n, k, packed)
        x_bits = synth.activations(m, k, cfg=60, mat=k)
        buf = torch.full((m * n + 64,), 12345.0, device="cuda")
        y = buf[32:32 + m * n]
        fp4.w4a16_midm(fmt, m, n, k, pw.q, pw.s, pw.global_scale, gc.x_tensor(x_bits), y)
        torch.cuda.synchronize()
        gc.check_product(fmt, packed, x_bits, y.view(m, n), label=f"midm {fmt} M={m} {n}x{k}")
        assert torch.all(buf[:32] == 12345.0) and torch.all(buf[32 + m * n:] == 12345.0)


@pytest.mark.parametrize("fmt", gc.FMTS)
def test_midm_one_hot_returns_weight_columns_exactly(fmt):
    n, k = 80, 384
    _announce("midm-one-hot", fmt)
    w, packed = gc.make_case(fmt, n, k, cfg=61)
    pw = gc.upload(fmt, n, k, packed)
    ks = np.arange(0, k, 7)[:50]
    x_bits = np.zeros((len(ks), k), np.uint16)
    x_bits[np.arange(len(ks)), ks] = 0x3F80
    y = torch.empty((len(ks), n), device="cuda")
    fp4.w4a16_midm(fmt, len(ks), n, k, pw.q, pw.s, pw.global_scale, gc.x_tensor(x_bits), y)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), ref.dequant_f32(fmt, packed)[:, ks].T)


def test_midm_repeatable():
    fmt, m, n, k = "rocmfp4_dual", 40, 96, 1024
    _announce("midm-repeat", fmt)
    w, packed = gc.make_case(fmt, n, k, cfg=62)
    pw = gc.upload(fmt, n, k, packed)
    x = gc.x_tensor(synth.activations(m, k, cfg=62))
    y1 = torch.empty((m, n), device="cuda")
    y2 = torch.empty((m, n), device="cuda")
    fp4.w4a16_midm(fmt, m, n, k, pw.q, pw.s, 1.0, x, y1)
    fp4.w4a16_midm(fmt, m, n, k, pw.q, pw.s, 1.0, x, y2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


# ------------------------------------------------------------------ GEMM

@pytest.mark.parametrize("fmt", gc.FMTS)
@pytest.mark.parametrize("m", [1, 17, 63, 64, 65, 100, 127, 128, 129, 191, 192, 193, 255, 256, 257, 383, 384, 511, 512, 513])
def test_gemm_shapes(fmt, m):
    for (n, k) in [(200, 384), (37, 160)]:
        _announce("gemm", fmt, m, n, k)
        w, packed = gc.make_case(fmt, n, k, cfg=55, mat=n)
        pw = gc.upload(fmt, n, k, packed)
        x_bits = synth.activations(m, k, cfg=55, mat=k)
        y = torch.full((m, n), float("nan"), device="cuda")
        fp4.w4a16_gemm(fmt, m, n, k, pw.q, pw.s, pw.global_scale, gc.x_tensor(x_bits), y)
        torch.cuda.synchronize()
        gc.check_product(fmt, packed, x_bits, y, label=f"gemm {fmt} M={m} {n}x{k}")


@pytest.mark.parametrize("fmt", gc.FMTS)
@pytest.mark.parametrize("k", [512, 640, 1152])
def test_gemm_multi_tile(fmt, k):
    # 2 x 3 output tiles with ragged last ones; K = 512, 640, 1152 give 8, 10 and 18 stages, which take the
    # stage loop's three-stage iterations, its single-stage remainder and the two peeled last stages
    m, n = 300, 600
    _announce("gemm-multi", fmt, m, n, k)
    w, packed = gc.make_case(fmt, n, k, cfg=57, mat=k)
    pw = gc.upload(fmt, n, k, packed)
    x_bits = synth.activations(m, k, cfg=57, mat=k + 1)
    y = torch.full((m, n), float("nan"), device="cuda")
    fp4.w4a16_gemm(fmt, m, n, k, pw.q, pw.s, pw.global_scale, gc.x_tensor(x_bits), y)
    torch.cuda.synchronize()
    gc.check_product(fmt, packed, x_bits, y, label=f"gemm-multi {fmt} M={m} {n}x{k}")


def test_gemm_short_tiles(tmp_path):
    # 7 x 37 tiles of 256 x 256 are between one and two rounds on a 256-CU GPU, so rows 0-1535 of every
    # column tile run as 192-row tiles (the rest as 256-row tiles); K = 672 is ragged. Sampled columns over
    # all rows against the oracle, and the whole output against the launch with 256-row tiles only
    # (FP4_GEMM_SHORT=0 in a child process; the same products in the same order: bitwise equal).
    m, n, k = 1792, 37 * 256, 672
    want = {}
    for fmt in gc.FMTS:
        _announce("gemm-short", fmt, m, n, k)
        w, packed = gc.make_case(fmt, n, k, cfg=61, mat=k)
        del w
        pw = gc.upload(fmt, n, k, packed)
        x_bits = synth.activations(m, k, cfg=61, mat=1)
        y = torch.full((m, n), float("nan"), device="cuda")
        fp4.w4a16_gemm(fmt, m, n, k, pw.q, pw.s, pw.global_scale, gc.x_tensor(x_bits), y)
        torch.cuda.synchronize()
        assert not torch.isnan(y).any()
        rng = np.random.default_rng(61)
        cols = np.unique(np.concatenate([[0, 255, 256, 8191, 8192, n - 1], rng.choice(n, 40, replace=False)]))
        gc.check_product(fmt, packed, x_bits, y, cols=cols, label=f"gemm-short {fmt}")
        gc.save_case(tmp_path, fmt, "gemm", fmt, m, n, k, pw, x_bits)
        want[fmt] = y.cpu().numpy()
    ys = gc.run_variant(tmp_path, {"FP4_GEMM_SHORT": "0"})
    for fmt, y in want.items():
        assert np.array_equal(y.view(np.uint32), ys[fmt].view(np.uint32)), fmt


def test_gemm_split_k(tmp_path):
    # Without a workspace (the C entry point w4a16_gemm), small grids (at most half as many tiles as CUs,
    # and not too many outputs) split K in two parts that add into the zeroed y: against the oracle,
    # repeatable to the bit (two addends onto zero give the same sum in either order), and the whole-K
    # launch (FP4_GEMM_SPLIT=0, in a child process) within the tolerance too.
    cases = {}
    for fmt in gc.FMTS:
        for (m, n, k) in [(100, 600, 1152), (256, 512, 2048), (257, 37, 4000)]:
            _announce("gemm-split", fmt, m, n, k)
            w, packed = gc.make_case(fmt, n, k, cfg=69, mat=k)
            pw = gc.upload(fmt, n, k, packed)
            x_bits = synth.activations(m, k, cfg=69, mat=m)
            x = gc.x_tensor(x_bits)
            ys = []
            for _ in range(3):
                y = torch.full((m, n), float("nan"), device="cuda")
                fp4.w4a16_gemm_noworkspace(fmt, m, n, k, pw.q, pw.s, pw.global_scale, x, y)
                ys.append(y)
            torch.cuda.synchronize()
            gc.check_product(fmt, packed, x_bits, ys[0], label=f"gemm-split {fmt} M={m} {n}x{k}")
            assert torch.equal(ys[0], ys[1]) and torch.equal(ys[0], ys[2])
            name = f"{fmt}_{m}_{n}_{k}"
            gc.save_case(tmp_path, name, "gemm", fmt, m, n, k, pw, x_bits)
            cases[name] = (fmt, packed, x_bits)
    whole = gc.run_variant(tmp_path, {"FP4_GEMM_SPLIT": "0"})
    for name, (fmt, packed, x_bits) in cases.items():
        gc.check_product(fmt, packed, x_bits, torch.from_numpy(whole[name]), label=f"gemm-whole {name}")


def test_gemm_band_row_tiles(tmp_path):
    # M <= 128 runs 128-row tiles, M <= 192 192-row tiles, and larger M on a small grid 128-row tiles over
    # several bands. Against the oracle as launched; and with one wave set per workgroup (FP4_GEMM_SETS=1, child
    # processes) the same products in the same order as the 256-row tiling (FP4_GEMM_BAND_ROWS=0), so those
    # outputs are bitwise equal (K = 1152 also takes the two-way split on both sides).
    n, k = 600, 1152
    want = {}
    for fmt in gc.FMTS:
        for m in (65, 128, 129, 192, 200, 256):
            _announce("gemm-band-rows", fmt, m, n, k)
            w, packed = gc.make_case(fmt, n, k, cfg=70, mat=m)
            pw = gc.upload(fmt, n, k, packed)
            x_bits = synth.activations(m, k, cfg=70, mat=m)
            y = torch.full((m, n), float("nan"), device="cuda")
            fp4.w4a16_gemm(fmt, m, n, k, pw.q, pw.s, pw.global_scale, gc.x_tensor(x_bits), y)
            torch.cuda.synchronize()
            gc.check_product(fmt, packed, x_bits, y, label=f"gemm-band-rows {fmt} M={m}")
            name = f"{fmt}_{m}"
            gc.save_case(tmp_path, name, "gemm", fmt, m, n, k, pw, x_bits)
            want[name] = y.cpu().numpy()
    bands = gc.run_variant(tmp_path, {"FP4_GEMM_SETS": "1"})
    ys = gc.run_variant(tmp_path, {"FP4_GEMM_SETS": "1", "FP4_GEMM_BAND_ROWS": "0"})
    for name in want:
        assert np.array_equal(bands[name].view(np.uint32), ys[name].view(np.uint32)), name


def test_gemm_narrow_tiles(tmp_path):
    # Grids of 256-column tiles that fill at most half the CUs run 128-column tiles (each wave owns 32 weight
    # rows), over 128-row bands where that grid fits the CUs. Against the oracle on sampled columns, and,
    # with K whole and one wave set per workgroup on both sides (FP4_GEMM_SPLIT=0, FP4_GEMM_SETS=1, child
    # processes: the two tilings may decide the split differently), bitwise against the 256-column tiling
    # (FP4_GEMM_NARROW=0): the same products in the same order. N = 1000 and 4350 leave a ragged last
    # 128-column tile.
    want = {}
    for fmt in gc.FMTS:
        for (m, n, k) in [(512, 4350, 2048), (300, 1000, 640), (700, 2304, 1024), (129, 1000, 1152)]:
            _announce("gemm-narrow", fmt, m, n, k)
            w, packed = gc.make_case(fmt, n, k, cfg=74, mat=m)
            pw = gc.upload(fmt, n, k, packed)
            x_bits = synth.activations(m, k, cfg=74, mat=m)
            y = torch.full((m, n), float("nan"), device="cuda")
            fp4.w4a16_gemm(fmt, m, n, k, pw.q, pw.s, pw.global_scale, gc.x_tensor(x_bits), y)
            torch.cuda.synchronize()
            assert not torch.isnan(y).any()
            cols = np.unique(np.concatenate([[0, 127, 128, n - 1], np.linspace(0, n - 1, 40).astype(int)]))
            gc.check_product(fmt, packed, x_bits, y, cols=cols, label=f"gemm-narrow {fmt} M={m} {n}x{k}")
            name = f"{fmt}_{m}_{n}_{k}"
            gc.save_case(tmp_path, name, "gemm", fmt, m, n, k, pw, x_bits)
            want[name] = y.cpu().numpy()
    narrow = gc.run_variant(tmp_path, {"FP4_GEMM_SPLIT": "0", "FP4_GEMM_SETS": "1"})
    wide = gc.run_variant(tmp_path, {"FP4_GEMM_SPLIT": "0", "FP4_GEMM_NARROW": "0", "FP4_GEMM_SETS": "1"})
    for name in want:
        assert np.array_equal(narrow[name].view(np.uint32), wide[name].view(np.uint32)), name


def test_gemm_two_wave_sets(tmp_path):
    # 128-row small-grid tiles run two sets of 4 waves over alternate stages, set 1's sums added to set 0's at
    # the end (also two 128-row bands for 128 < M <= 192). K from 2 stages (one per set) up, ragged K = 672,
    # split and whole K: against the oracle as launched, bitwise repeatable, and against the oracle again with
    # one set (FP4_GEMM_SETS=1), with K forced whole (FP4_GEMM_SPLIT=0), with the two-part atomic split
    # forced wherever the grid allows (FP4_GEMM_SPLIT=1, FP4_GEMM_PARTS=1) and with two K parts in the
    # workspace (FP4_GEMM_PARTS=2).
    shapes = [(65, 1000, 128), (65, 1000, 256), (100, 600, 1152), (128, 2304, 1024), (256, 600, 672),
              (200, 1000, 640), (97, 14336, 256), (160, 2304, 1152), (192, 1000, 384)]
    cases = {}
    for fmt in gc.FMTS:
        for (m, n, k) in shapes:
            _announce("gemm-sets", fmt, m, n, k)
            w, packed = gc.make_case(fmt, n, k, cfg=76, mat=k + m)
            del w
            pw = gc.upload(fmt, n, k, packed)
            x_bits = synth.activations(m, k, cfg=76, mat=k + m)
            x = gc.x_tensor(x_bits)
            ys = []
            for _ in range(2):
                y = torch.full((m, n), float("nan"), device="cuda")
                fp4.w4a16_gemm(fmt, m, n, k, pw.q, pw.s, pw.global_scale, x, y)
                ys.append(y)
            torch.cuda.synchronize()
            assert torch.equal(ys[0], ys[1])
            cols = np.unique(np.concatenate([[0, 127, 128, n - 1], np.linspace(0, n - 1, 24).astype(int)]))
            gc.check_product(fmt, packed, x_bits, ys[0], cols=cols, label=f"gemm-sets {fmt} M={m} {n}x{k}")
            name = f"{fmt}_{m}_{n}_{k}"
            gc.save_case(tmp_path, name, "gemm", fmt, m, n, k, pw, x_bits)
            cases[name] = (fmt, packed, x_bits, cols)
    for env in ({"FP4_GEMM_SETS": "1"}, {"FP4_GEMM_SPLIT": "0"}, {"FP4_GEMM_SPLIT": "1", "FP4_GEMM_PARTS": "1"},
                {"FP4_GEMM_PARTS": "2"}):
        ys = gc.run_variant(tmp_path, env)
        for name, (fmt, packed, x_bits, cols) in cases.items():
            gc.check_product(fmt, packed, x_bits, torch.from_numpy(ys[name]), cols=cols, label=f"{env} {name}")


def test_gemm_k_parts():
    # Grids that leave CUs idle (small N, long K) split K into P parts written to a workspace and added in a
    # fixed order by a second kernel: the 2560 x 9728 projection at M = 65, 128 and 200 (20 or 40 tiles), the
    # 9728 x 2560 one at M = 96, 4096 x 4096 at M = 128 and a ragged K. Against the oracle on sampled columns
    # with the workspace the library asks for, bitwise repeatable; with a workspace for two planes only (the
    # largest split that fits), and with none (the C entry point w4a16_gemm), against the oracle too.
    shapes = [(65, 2560, 9728), (128, 2560, 9728), (200, 2560, 9728), (96, 9728, 2560), (128, 4096, 4096),
              (100, 1000, 4000)]
    for fmt in gc.FMTS:
        for (m, n, k) in shapes:
            _announce("gemm-k-parts", fmt, m, n, k)
            assert fp4.w4a16_gemm_workspace_bytes(fmt, m, n, k) > 2 * m * n * 4   # more than two parts
            w, packed = gc.make_case(fmt, n, k, cfg=77, mat=k + m)
            del w
            pw = gc.upload(fmt, n, k, packed)
            x_bits = synth.activations(m, k, cfg=77, mat=k + m)
            x = gc.x_tensor(x_bits)
            cols = np.unique(np.concatenate([[0, 127, 128, n - 1], np.linspace(0, n - 1, 24).astype(int)]))
            ys = []
            for _ in range(2):
                y = torch.full((m, n), float("nan"), device="cuda")
                fp4.w4a16_gemm(fmt, m, n, k, pw.q, pw.s, pw.global_scale, x, y)
                ys.append(y)
            small = torch.empty(2 * m * n * 4, dtype=torch.uint8, device="cuda")
            y2 = torch.full((m, n), float("nan"), device="cuda")
            fp4.w4a16_gemm(fmt, m, n, k, pw.q, pw.s, pw.global_scale, x, y2, workspace=small)
            y0 = torch.full((m, n), float("nan"), device="cuda")
            fp4.w4a16_gemm_noworkspace(fmt, m, n, k, pw.q, pw.s, pw.global_scale, x, y0)
            torch.cuda.synchronize()
            assert torch.equal(ys[0], ys[1])
            for lab, yy in (("parts", ys[0]), ("two planes", y2), ("no workspace", y0)):
                gc.check_product(fmt, packed, x_bits, yy, cols=cols, label=f"gemm-k-parts {lab} {fmt} M={m} {n}x{k}")


def test_gemm_small_grid_stage_counts():
    # The small-grid kernels (128-column tiles of 128, 192 and 256 rows) over K of 2 to 24 stages (K = 672
    # ragged): a K loop with no full ring period, the single-stage remainder and both peeled last stages; from
    # 12 stages K also splits in two parts at stage 3 floor(H / 6) of H. Against the oracle on sampled
    # columns.
    shapes = ([(65, 1000, k) for k in (128, 256, 384, 512, 672, 768, 1024, 1536)] +
              [(150, 600, k) for k in (256, 896, 1152)] + [(300, 11008, k) for k in (128, 256, 384, 640, 1024)])
    for fmt in gc.FMTS:
        for (m, n, k) in shapes:
            _announce("gemm-stage-counts", fmt, m, n, k)
            w, packed = gc.make_case(fmt, n, k, cfg=75, mat=k + m)
            del w
            pw = gc.upload(fmt, n, k, packed)
            x_bits = synth.activations(m, k, cfg=75, mat=k + m)
            y = torch.full((m, n), float("nan"), device="cuda")
            fp4.w4a16_gemm(fmt, m, n, k, pw.q, pw.s, pw.global_scale, gc.x_tensor(x_bits), y)
            torch.cuda.synchronize()
            assert not torch.isnan(y).any()
            cols = np.unique(np.concatenate([[0, 127, 128, n - 1], np.linspace(0, n - 1, 24).astype(int)]))
            gc.check_product(fmt, packed, x_bits, y, cols=cols, label=f"gemm-stages {fmt} M={m} {n}x{k}")


@pytest.mark.parametrize("entry", ["w4a16_gemm_noworkspace", "w4a16_gemm"])
def test_gemm_split_in_graph(entry):
    # The split-K GEMM enqueues a zero-fill kernel and the product (no workspace), or the K parts into a
    # workspace (allocated by the binding inside the capture) and the kernel that adds them: captured in a
    # graph (on torch's capture stream) and replayed several times, with eager work and synchronizations
    # between the replays, every replay gives the eager result bit for bit.
    fmt, m, n, k = "rocmfp4_fast", 128, 512, 2048
    _announce("gemm-split-graph", entry, fmt, m, n, k)
    fn = getattr(fp4, entry)
    w, packed = gc.make_case(fmt, n, k, cfg=71)
    pw = gc.upload(fmt, n, k, packed)
    x = gc.x_tensor(synth.activations(m, k, cfg=71))
    if entry == "w4a16_gemm":
        assert fp4.w4a16_gemm_workspace_bytes(fmt, m, n, k) > 0   # the K-parts path
    y_eager = torch.full((m, n), float("nan"), device="cuda")
    fn(fmt, m, n, k, pw.q, pw.s, pw.global_scale, x, y_eager)
    torch.cuda.synchronize()
    y = torch.full((m, n), float("nan"), device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn(fmt, m, n, k, pw.q, pw.s, pw.global_scale, x, y)
    for rep in range(4):
        y.fill_(float("nan") if rep % 2 else 7.0)
        junk = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {rep} differs"
        del junk


@pytest.mark.parametrize("fmt", gc.FMTS)
def test_gemm_identity_returns_weights_exactly(fmt):
    # x = I (M = K) gives y = W32^T exactly
    n, k = 96, 256
    _announce("gemm-identity", fmt)
    w, packed = gc.make_case(fmt, n, k, cfg=56)
    pw = gc.upload(fmt, n, k, packed)
    x_bits = np.zeros((k, k), np.uint16)
    x_bits[np.arange(k), np.arange(k)] = 0x3F80
    y = torch.empty((k, n), device="cuda")
    fp4.w4a16_gemm(fmt, k, n, k, pw.q, pw.s, pw.global_scale, gc.x_tensor(x_bits), y)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), ref.dequant_f32(fmt, packed).T)


@pytest.mark.parametrize("m", [1, 16, 17, 40, 64, 65])
def test_matmul_dispatch(m):
    fmt, n, k = "nvfp4", 64, 256
    _announce("matmul", m)
    w, packed = gc.make_case(fmt, n, k, cfg=57)
    pw = gc.upload(fmt, n, k, packed)
    x_bits = synth.activations(m, k, cfg=57)
    y = pw.matmul(gc.x_tensor(x_bits))
    torch.cuda.synchronize()
    gc.check_product(fmt, packed, x_bits, y, label=f"matmul M={m}")


def test_matmul_gemm_band():
    # 48 <= M <= 64 on matrices of at least 20 M weights: with a workspace that holds its K parts,
    # w4a16_matmul_ws runs the GEMM (the binding provides the workspace); with a smaller one, the mid-M kernel
    # (bitwise what w4a16_midm gives). Both against the oracle on sampled columns.
    for fmt in ("nvfp4", "rocmfp4_dual"):
        for (m, n, k) in [(48, 2560, 9728), (64, 9728, 2560)]:
            _announce("matmul-gemm-band", fmt, m, n, k)
            need = fp4.w4a16_matmul_workspace_bytes(fmt, m, n, k)
            assert need == fp4.w4a16_gemm_workspace_bytes(fmt, m, n, k) > 0
            w, packed = gc.make_case(fmt, n, k, cfg=79, mat=m)
            del w
            pw = gc.upload(fmt, n, k, packed)
            x_bits = synth.activations(m, k, cfg=79, mat=m)
            x = gc.x_tensor(x_bits)
            y = torch.full((m, n), float("nan"), device="cuda")
            fp4.w4a16_matmul(fmt, m, n, k, pw.q, pw.s, pw.global_scale, x, y)
            y_small = torch.full((m, n), float("nan"), device="cuda")
            fp4.w4a16_matmul(fmt, m, n, k, pw.q, pw.s, pw.global_scale, x, y_small,
                             workspace=torch.empty(need // 2, dtype=torch.uint8, device="cuda"))
            y_midm = torch.full((m, n), float("nan"), device="cuda")
            fp4.w4a16_midm(fmt, m, n, k, pw.q, pw.s, pw.global_scale, x, y_midm)
            torch.cuda.synchronize()
            assert torch.equal(y_small, y_midm)
            cols = np.unique(np.concatenate([[0, n - 1], np.linspace(0, n - 1, 24).astype(int)]))
            for lab, yy in (("gemm", y), ("midm", y_small)):
                gc.check_product(fmt, packed, x_bits, yy, cols=cols, label=f"matmul-band {lab} {fmt} M={m} {n}x{k}")


def _random_shapes(fmt, count, seed):
    # Seeded shapes across all three product paths (GEMV M <= 16, mid-M 17..64, GEMM above), with ragged
    # N (any value) and K (any multiple of the format's block), so tile and chunk tails land anywhere.
    rng = np.random.default_rng(seed)
    kmul = 16 if fmt == "nvfp4" else 32
    bands = [(1, 16)] if fmt == "q4_0" else [(1, 16), (17, 64), (65, 300)]
    out = []
    for i in range(count):
        lo, hi = bands[i % len(bands)]
        out.append((int(rng.integers(lo, hi + 1)), int(rng.integers(1, 641)), kmul * int(rng.integers(1, 2560 // kmul + 1))))
    return out


@pytest.mark.parametrize("fmt", gc.FMTS_ALL)
def test_matmul_random_shapes(fmt):
    for case, (m, n, k) in enumerate(_random_shapes(fmt, 9, seed=1000 + gc.FMTS_ALL.index(fmt))):
        _announce("matmul-random", fmt, m, n, k)
        w, packed = gc.make_case(fmt, n, k, cfg=67, mat=case)
        pw = gc.upload(fmt, n, k, packed)
        x_bits = synth.activations(m, k, cfg=67, mat=case)
        y = torch.full((m, n), float("nan"), device="cuda")
        fp4.w4a16_matmul(fmt, m, n, k, pw.q, pw.s, pw.global_scale, gc.x_tensor(x_bits), y)
        torch.cuda.synchronize()
        gc.check_product(fmt, packed, x_bits, y, label=f"matmul {fmt} M={m} N={n} K={k}")


# ------------------------------------------------------------------ device packers (byte-exact)

@pytest.mark.parametrize("fmt", gc.FMTS_ALL)
@pytest.mark.parametrize("dist,outl", [("t", 0.0), ("t", 0.001), ("normal", 0.0)])
def test_device_packer_matches_oracle(fmt, dist, outl):
    n, k = 64, 512
    _announce("quantize", fmt, dist, outl)
    w = synth.weights(n, k, dist=dist, nu=4.0, outlier_frac=outl, cfg=58)
    want = pack.pack(fmt, w)
    wt = torch.from_numpy(w).cuda()
    if fmt == "nvfp4":
        wq = torch.empty(n * k // 2, dtype=torch.uint8, device="cuda")
        ws = torch.empty(n * k // 16, dtype=torch.uint8, device="cuda")
        g = torch.empty(1, device="cuda")
        fp4.fp4_quantize_nvfp4(n, k, wt, wq, ws, g)
        torch.cuda.synchronize()
        assert np.array_equal(wq.cpu().numpy().reshape(n, -1), want[0])
        assert np.array_equal(ws.cpu().numpy().reshape(n, -1), want[1])
        assert g.item() == want[2]
    else:
        bb = layouts.BLOCK_BYTES[fmt]
        blocks = torch.empty(n * (k // 32) * bb, dtype=torch.uint8, device="cuda")
        if fmt == "q4_0":
            fp4.fp4_quantize_q4_0(n, k, wt, blocks)
        else:
            fp4.fp4_quantize_rocmfp4(fmt, n, k, wt, None, blocks)
        torch.cuda.synchronize()
        assert np.array_equal(blocks.cpu().numpy().reshape(n, k // 32, bb), want[0])


@pytest.mark.parametrize("fmt", ["rocmfp4_dual", "rocmfp4_fast"])
def test_device_packer_importance(fmt):
    n, k = 16, 256
    _announce("quantize-importance", fmt)
    w = synth.weights(n, k, dist="t", nu=4.0, outlier_frac=0.01, cfg=59)
    v = np.abs(synth.weights(n, k, dist="normal", sigma=1.0, cfg=59, mat=1)).astype(np.float32)
    want = pack.pack(fmt, w, importance=v)
    blocks = torch.empty(n * (k // 32) * layouts.BLOCK_BYTES[fmt], dtype=torch.uint8, device="cuda")
    fp4.fp4_quantize_rocmfp4(fmt, n, k, torch.from_numpy(w).cuda(), torch.from_numpy(v).cuda(), blocks)
    torch.cuda.synchronize()
    assert np.array_equal(blocks.cpu().numpy().reshape(want[0].shape), want[0])


def test_device_packer_edge_values():
    # zeros, exact ties on every E2M1 / Codebook10 midpoint, a huge and a tiny block
    n, k = 16, 128
    w = np.zeros((n, k), np.float32)
    w[0, :7] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]) * 448 / 6 * 2  # NVFP4 ties at d
    w[1, :16] = 2688.0 * np.linspace(-1, 1, 16)
    w[2, :32] = np.array([0.5, 1.5, 2.5, 3.5, 5, 7, 9] * 4 + [10, 11, 12, 13], np.float32)
    w[3, :32] = 1e-6
    w[4, 16:48] = -3e-3
    w[5, :32] = np.array([-2.0, 1.0, 0.125, 0.25, 0.375, 1.75, -1.75] + [0.0] * 25, np.float32)  # Q4_0 halves
    w[6, :32] = 7.0
    w[6, 5] = -7.0                                   # equal magnitudes: the first (+7) decides the sign
    for fmt in gc.FMTS_ALL:
        _announce("quantize-edges", fmt)
        want = pack.pack(fmt, w)
        wt = torch.from_numpy(w).cuda()
        if fmt == "nvfp4":
            wq = torch.empty(n * k // 2, dtype=torch.uint8, device="cuda")
            ws = torch.empty(n * k // 16, dtype=torch.uint8, device="cuda")
            g = torch.empty(1, device="cuda")
            fp4.fp4_quantize_nvfp4(n, k, wt, wq, ws, g)
            torch.cuda.synchronize()
            assert np.array_equal(wq.cpu().numpy().reshape(n, -1), want[0])
            assert np.array_equal(ws.cpu().numpy().reshape(n, -1), want[1])
            assert g.item() == want[2]
        else:
            bb = layouts.BLOCK_BYTES[fmt]
            blocks = torch.empty(n * (k // 32) * bb, dtype=torch.uint8, device="cuda")
            if fmt == "q4_0":
                fp4.fp4_quantize_q4_0(n, k, wt, blocks)
            else:
                fp4.fp4_quantize_rocmfp4(fmt, n, k, wt, None, blocks)
            torch.cuda.synchronize()
            assert np.array_equal(blocks.cpu().numpy().reshape(n, k // 32, bb), want[0])
    # all-zero matrix: g = 1 and zero codes
    wq = torch.empty(n * k // 2, dtype=torch.uint8, device="cuda")
    ws = torch.empty(n * k // 16, dtype=torch.uint8, device="cuda")
    g = torch.empty(1, device="cuda")
    fp4.fp4_quantize_nvfp4(n, k, torch.zeros(n, k, device="cuda"), wq, ws, g)
    torch.cuda.synchronize()
    assert g.item() == 1.0 and not wq.any() and not ws.any()
