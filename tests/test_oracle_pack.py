"""Pins of the oracle's packers: exact rational brute force, worked cases, invariants (CPU)."""
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import synth
from oracle import formats, layouts, pack, ref
from tests import golden_io

LEVELS = [0, 1, 2, 3, 4, 6, 8, 10]
E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]
UE4M3 = [Fraction(float(v)) for v in formats.E4M3_POSITIVE_GRID]


def _nearest_index(x: Fraction, grid) -> int:
    """Nearest grid point by exact distance; ties to the even index."""
    best, bd = 0, None
    for i, v in enumerate(grid):
        d = abs(x - v)
        if bd is None or d < bd or (d == bd and i % 2 == 0):
            best, bd = i, d
    return best


def _exact_errors(w, s_list=UE4M3):
    """Exact E(c) = sum (|w| - L s)^2 for every candidate, L the exact nearest level (ties even)."""
    ws = [abs(Fraction(float(v))) for v in w]
    out = []
    for s in s_list:
        e = Fraction(0)
        for a in ws:
            L = 0 if s == 0 else LEVELS[_nearest_index(a / s, [Fraction(l) for l in LEVELS])]
            e += (a - L * s) ** 2
        out.append(e)
    return out


finite_f32 = st.floats(min_value=-50.0, max_value=50.0, allow_nan=False, allow_infinity=False, width=32)


@settings(max_examples=60, deadline=None)
@given(st.lists(finite_f32, min_size=1, max_size=8))
def test_search_selects_exact_minimum(ws):
    w = np.array(ws, dtype=np.float32)
    codes, scales, errs = pack.rocmfp4_search(w[None, :])
    exact = _exact_errors(w)
    emin = min(exact)
    c = int(scales[0])
    # the chosen candidate's exact error is the exact minimum up to FP64 rounding of the sum
    tol = Fraction(2 ** -48) * (sum(abs(Fraction(float(v))) for v in w) ** 2 + 1) * len(w)
    assert exact[c] - emin <= tol * (emin + Fraction(1, 10 ** 30)) or exact[c] == emin
    # the codes are the exact nearest levels at the chosen scale, with the sign rule
    s = UE4M3[c]
    for wi, code in zip(w, codes[0]):
        L = 0 if s == 0 else _nearest_index(abs(Fraction(float(wi))) / s, [Fraction(l) for l in LEVELS])
        assert code & 7 == L
        assert (code >> 3) == (1 if (wi < 0 and L != 0) else 0)


@settings(max_examples=30, deadline=None)
@given(st.lists(st.floats(min_value=-3.0, max_value=3.0, allow_nan=False, width=32), min_size=16, max_size=16))
def test_search_invariants(ws):
    w = np.array(ws, dtype=np.float32)
    _, scales, errs = pack.rocmfp4_search(w[None, :])
    all_e = pack.rocmfp4_all_errors(w[None, :])[0]
    c = int(scales[0])
    assert errs[0] == all_e[c] == all_e.min()
    a = float(np.max(np.abs(w)))
    start = int(formats.e4m3_encode_rne(min(a / 10, 448.0)))
    assert all_e[c] <= all_e[start]
    # the max-preserving candidate: the smallest scale with 10 s >= max|w|
    mp = next((i for i in range(127) if 10 * formats.E4M3_POSITIVE_GRID[i] >= a), 126)
    assert all_e[c] <= all_e[mp]
    # among equal errors the candidate closest to the start wins (lower code on a tie)
    best = [i for i in range(127) if all_e[i] == all_e.min()]
    assert c == min(best, key=lambda i: (abs(i - start), i))


def test_clipping_can_win():
    # 15 calm weights at 1.0 and one outlier at 10.5: scale 1.0 clips the outlier to 10 (error 0.25)
    # and beats the max-preserving scale 1.125, which moves every calm weight (error ~0.80)
    w = np.array([1.0] * 15 + [10.5], dtype=np.float32)
    _, scales, _ = pack.rocmfp4_search(w[None, :])
    s = formats.ue4m3_value(scales[0])
    all_e = pack.rocmfp4_all_errors(w[None, :])[0]
    mp = next(i for i in range(127) if 10 * formats.E4M3_POSITIVE_GRID[i] >= 10.5)
    assert s == 1.0 and 10 * s < 10.5
    assert all_e[scales[0]] == 0.25 and all_e[scales[0]] < all_e[mp]


def test_search_worked_case():
    g = golden_io.read("hand_packed.txt")
    scale = int(g["search_scale"][0], 16)
    w = np.array([float(v) for v in g["search_levels"]], dtype=np.float64) * float(formats.ue4m3_value(scale))
    codes, scales, errs = pack.rocmfp4_search(w.astype(np.float32)[None, :])
    assert scales[0] == scale and errs[0] == 0.0
    assert codes[0].tolist() == golden_io.hex_bytes(g["search_codes"])


def test_empty_group_selects_zero_code():
    g = golden_io.read("widget_defaults.txt")
    codes, scales, errs = pack.rocmfp4_search(np.zeros((1, 16), np.float32))
    assert scales[0] == int(g["empty_group_selected"][0], 16) and errs[0] == 0 and not codes.any()


def test_widget_snap_and_error():
    # normalized grid (scale 1.0 = UE4M3 0x38): a probe 0.3 from 3 snaps to 3 with error 0.3
    g = golden_io.read("widget_defaults.txt")
    level, err = float(g["snap_level"][0]), float(g["snap_error"][0])
    for probe in (level + err, level - err):
        e = pack.rocmfp4_all_errors(np.array([[probe]], np.float32))[0, 0x38]
        assert e == pytest.approx(err ** 2, rel=1e-6)
        # and the stock uniform integer grid snaps the same way
        assert round(probe) == level and abs(probe - round(probe)) == pytest.approx(err)


def test_importance_weighting_moves_the_choice():
    # an outlier with zero importance is ignored: the fit matches the other 15 exactly
    w = np.full(16, 0.8125 * 3, np.float32)
    w[5] = 0.8125 * 13                       # not representable at 0.8125 (clips to 10)
    v = np.ones(16, np.float32)
    v[5] = 0.0
    _, s_w, e_w = pack.rocmfp4_search(w[None, :], v[None, :])
    assert e_w[0] == 0.0
    _, s_u, e_u = pack.rocmfp4_search(w[None, :])
    assert e_u[0] > 0.0


def test_dual_and_fast_groups():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((3, 64)) * 0.02).astype(np.float32)
    blocks, g = pack.pack_rocmfp4("rocmfp4_dual", w)
    assert blocks.shape == (3, 2, 18) and g == 1.0
    codes, sc = layouts.rocm_split("rocmfp4_dual", blocks)
    c2, s2, _ = pack.rocmfp4_search(w.reshape(-1, 16))
    assert np.array_equal(sc.reshape(-1), s2) and np.array_equal(codes.reshape(-1, 16), c2)
    blocks, _ = pack.pack_rocmfp4("rocmfp4_fast", w)
    assert blocks.shape == (3, 2, 17)
    codes, sc = layouts.rocm_split("rocmfp4_fast", blocks)
    c3, s3, _ = pack.rocmfp4_search(w.reshape(-1, 32))
    assert np.array_equal(sc.reshape(-1), s3) and np.array_equal(codes.reshape(-1, 32), c3)


# ------------------------------- NVFP4 RTN -------------------------------------

def test_nvfp4_worked_case():
    g = golden_io.read("hand_packed.txt")
    w = np.zeros((1, 32), np.float32)
    w[0, :3] = [2688, -1344, 672]
    w[0, 16:20] = [6, -3, 1.5, 0.5]
    wq, ws, gs = pack.pack_nvfp4(w)
    assert gs == float(g["rtn_g"][0])
    assert ws[0].tolist() == golden_io.hex_bytes(g["rtn_scales"])
    assert layouts.nvfp4_split(wq)[0].tolist() == golden_io.hex_bytes(g["rtn_codes"])


@settings(max_examples=40, deadline=None)
@given(st.lists(st.floats(min_value=-1e3, max_value=1e3, allow_nan=False, width=32), min_size=32, max_size=32))
def test_nvfp4_rtn_bruteforce(ws):
    w = np.array(ws, dtype=np.float32).reshape(1, 32)
    wq, wsc, g = pack.pack_nvfp4(w)
    amax = float(np.max(np.abs(w)))
    if amax == 0 or float(np.float32(amax) / np.float32(2688)) == 0:
        assert not wq.any() and g == 1.0
        return
    assert g == np.float32(float(Fraction(amax) / 2688))           # single rounding of amax / 2688
    codes = layouts.nvfp4_split(wq)[0]
    for b in range(2):
        blk = w[0, 16 * b:16 * b + 16]
        q = float(np.max(np.abs(blk))) / (6.0 * float(g))            # the FP64 quotient
        want_s = 126 if q >= 448 else _nearest_index(Fraction(q), UE4M3[:127])
        assert wsc[0, b] == want_s
        d = UE4M3[want_s] * Fraction(float(g))
        for i, wi in enumerate(blk):
            c = codes[16 * b + i]
            L = 0 if d == 0 else _nearest_index(abs(Fraction(float(wi))) / d, E2M1)
            assert c & 7 == L
            assert (c >> 3) == (1 if (wi < 0 and L != 0) else 0)


def test_nvfp4_amax_block_gets_max_scale():
    rng = np.random.default_rng(4)
    w = rng.standard_t(5, size=(32, 128)).astype(np.float32) * 0.02
    wq, ws, g = pack.pack_nvfp4(w)
    i = np.unravel_index(np.argmax(np.abs(w)), w.shape)
    assert ws[i[0], i[1] // 16] == 0x7E
    assert layouts.nvfp4_split(wq)[i] & 7 == 7
    w64 = ref.dequant("nvfp4", (wq, ws, g))
    assert abs(w64[i]) == pytest.approx(abs(float(w[i])), rel=1e-6)


def test_nvfp4_all_zero():
    wq, ws, g = pack.pack_nvfp4(np.zeros((2, 32), np.float32))
    assert g == 1.0 and not wq.any() and not ws.any()


def test_level_ties_go_to_even_code():
    # weights exactly on every midpoint of Codebook10 at scale 1.0 (UE4M3 0x38)
    mids = [0.5, 1.5, 2.5, 3.5, 5.0, 7.0, 9.0]
    want = [0, 2, 2, 4, 4, 6, 6]                 # the even code of each neighbouring pair
    all_e = pack.rocmfp4_all_errors(np.array([[m] for m in mids], np.float32))[:, 0x38]
    for m, c, e in zip(mids, want, all_e):
        assert e == (m - LEVELS[c]) ** 2
    # NVFP4: every E2M1 midpoint times d = e4m3(0x38) * g, with g = 1 (amax = 2688 elsewhere in the row)
    w = np.zeros((1, 32), np.float32)
    w[0, 0] = 2688.0
    w[0, 16] = 6.0                               # block 1 scale -> 1.0
    e2m1_mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    w[0, 17:24] = e2m1_mids
    wq, ws, g = pack.pack_nvfp4(w)
    assert g == 1.0 and ws[0, 1] == 0x38
    assert layouts.nvfp4_split(wq)[0, 17:24].tolist() == [0, 2, 2, 4, 4, 6, 6]


# ---------------------------------------------------------------- Q4_0 (signed abs-max)

def test_q4_0_worked_case():
    g = golden_io.read("hand_packed.txt")
    w = np.zeros((1, 32), np.float32)
    w[0, :8] = golden_io.floats(g["q4_0_pack_weights"])
    blocks, gs = pack.pack_q4_0(w)
    assert gs == 1.0
    assert blocks[0, 0, :2].tolist() == golden_io.hex_bytes(g["q4_0_pack_scale_bytes"])
    codes, _ = layouts.q4_0_split(blocks)
    assert codes[0].tolist() == golden_io.hex_bytes(g["q4_0_pack_codes"])


def test_q4_0_signed_absmax_maps_extreme_to_grid_end():
    # the largest-magnitude weight (sign kept) always gets code 0, i.e. level -8; when m / -8 is an
    # FP16 value it is reconstructed exactly
    rng = np.random.default_rng(21)
    w = (rng.standard_normal((40, 64)) * 0.02).astype(np.float32)
    w[3, 5] = 0.25                      # positive extreme: d = -0.03125, exact in FP16
    w[7, 40] = -0.5                     # negative extreme: d = 0.0625
    blocks, _ = pack.pack_q4_0(w)
    codes, d = layouts.q4_0_split(blocks)
    b = w.reshape(-1, 32).astype(np.float64)
    first = np.argmax(np.abs(b), axis=1)
    assert np.all(codes.reshape(-1, 32)[np.arange(b.shape[0]), first] == 0)
    w64 = ref.dequant("q4_0", (blocks, np.float32(1)))
    assert w64[3, 5] == 0.25 and w64[7, 40] == -0.5


def test_q4_0_codes_are_nearest_level_bruteforce():
    # every code is the level nearest w / d (exact rationals), a tie taking the larger level
    rng = np.random.default_rng(22)
    w = (rng.standard_t(4, (6, 64)) * 0.05).astype(np.float32)
    w[0, 1] = w[0, 0] * np.float32(-0.0625)   # exactly half a step: w / d = 0.5
    blocks, _ = pack.pack_q4_0(w)
    codes, _ = layouts.q4_0_split(blocks)
    bw = w.reshape(-1, 32)
    bc = codes.reshape(-1, 32)
    for r in range(bw.shape[0]):
        a = [Fraction(float(v)) for v in bw[r]]
        m = max(a, key=abs)
        m = next(v for v in a if abs(v) == abs(m))          # first of the largest magnitude
        d = m / -8
        for v, c in zip(a, bc[r]):
            if d == 0:
                assert c == 8
                continue
            best = min(range(16), key=lambda q: (abs(v - (q - 8) * d), -q))
            assert c == best, (r, v, c, best)


def test_q4_0_zero_block():
    blocks, _ = pack.pack_q4_0(np.zeros((2, 32), np.float32))
    codes, d = layouts.q4_0_split(blocks)
    assert np.all(codes == 8) and np.all(d == 0)


def test_nvfp4_row_sample_packs_like_the_whole_matrix():
    # rows are packed independently once the whole-matrix global scale is known, so packing a row
    # sample with that scale gives exactly those rows of the whole matrix's bytes
    w = synth.weights(48, 128, dist="t", nu=5.0, cfg=96)
    wq, ws, g = pack.pack_nvfp4(w)
    rows = np.array([0, 7, 8, 31, 47])
    sq, ss, sg = pack.pack_nvfp4_rows(w[rows], pack.nvfp4_global_scale(w))
    assert sg == g
    assert np.array_equal(sq, wq[rows]) and np.array_equal(ss, ws[rows])
    # a sample packed on its own would take its own (smaller) amax: different bytes in general
    assert pack.nvfp4_global_scale(w[rows]) <= g
