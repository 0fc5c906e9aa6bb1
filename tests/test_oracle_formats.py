"""Pins of the oracle's codecs and layouts against the pages and independent decoders (CPU)."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats, layouts
from tests import golden_io


def test_codebook10_levels_match_page():
    g = golden_io.read("codebook10.txt")
    levels = golden_io.floats(g["levels"])
    assert list(formats.CODEBOOK10_MAGNITUDE) == levels
    vals = formats.codebook10_value(np.arange(16))
    # the signed grid is exactly 0, +-1, +-2, +-3, +-4, +-6, +-8, +-10
    assert sorted(set(vals.tolist())) == sorted(set(levels) | {-v for v in levels})
    assert vals[8] == 0.0 and not np.signbit(vals[8])      # code 8 is level 0


def test_codebook10_is_e2m1_derived_with_outer_retuned():
    g = golden_io.read("codebook10.txt")
    for c in range(16):
        if c & 7 == 7:
            assert formats.codebook10_value(c) == np.copysign(float(g["outer_after_retune"][0]),
                                                             -1 if c & 8 else 1)
            assert 2 * abs(formats.e2m1_value(c)) == float(g["e2m1_derived_outer_before_retune"][0])
        else:
            assert abs(formats.codebook10_value(c)) == 2 * abs(formats.e2m1_value(c))


def test_e2m1_table():
    # OCP FP4 E2M1: sign, 2-bit exponent (bias 1), 1-bit mantissa; exponent 0 is subnormal (0, 0.5)
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        v = (m * 0.5) if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)
        want = -v if s else v
        got = formats.e2m1_value(c)
        assert got == want and np.signbit(got) == bool(s)


def test_e4m3_all_bytes_vs_torch():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = formats.e4m3_value(b)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))
    assert formats.e4m3_value(0x7E) == 448.0 and formats.e4m3_value(1) == 2.0 ** -9


def test_ue4m3_masks_sign_and_has_127_finite_candidates():
    b = np.arange(256)
    assert np.array_equal(formats.ue4m3_value(b)[:128], formats.ue4m3_value(b + 128)[:128], equal_nan=True)
    finite = np.isfinite(formats.ue4m3_value(np.arange(128)))
    assert finite.sum() == 127 and not finite[0x7F]
    assert np.all(np.diff(formats.E4M3_POSITIVE_GRID) > 0)


def test_widget_half_scales_decode_from_ue4m3():
    # the lab displays three decimals; exactly one UE4M3 code displays as each value
    g = golden_io.read("widget_defaults.txt")
    grid = formats.E4M3_POSITIVE_GRID

    def display(v):  # round half up to three decimals, on the exact binary value
        return int(Fraction(v) * 1000 + Fraction(1, 2)) / 1000

    for shown, code in zip(golden_io.floats(g["half_scales_display"]), (0x35, 0x1C)):
        matches = [c for c in range(127) if display(grid[c]) == shown]
        assert matches == [code]


def _nearest_e4m3_bruteforce(v: float) -> int:
    fv = Fraction(v)
    best, best_d = None, None
    for c in range(127):
        d = abs(Fraction(float(formats.E4M3_POSITIVE_GRID[c])) - fv)
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best


def test_e4m3_encode_rne_bruteforce():
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        rng.uniform(0, 460, 300), np.exp2(rng.uniform(-12, 9, 300)),
        formats.E4M3_POSITIVE_GRID,
        (formats.E4M3_POSITIVE_GRID[1:] + formats.E4M3_POSITIVE_GRID[:-1]) / 2,  # exact ties
        [0.0, 447.9, 448.0, 460.0, 1e9, 2.0 ** -11, 2.0 ** -10],
    ])
    got = formats.e4m3_encode_rne(vals)
    for v, c in zip(vals, got):
        want = 126 if v >= 448 else _nearest_e4m3_bruteforce(float(v))
        assert c == want, (v, c, want)


def test_block_densities_match_page():
    g = golden_io.read("block_density.txt")
    for fmt in ("rocmfp4_dual", "rocmfp4_fast", "nvfp4", "q4_0"):
        wpb, bb, bpw, group, nscale = g[fmt]
        assert layouts.canonical_bytes(fmt, 1, 32) * int(wpb) == int(bb) * 32
        assert layouts.bits_per_weight(fmt) == pytest.approx(float(bpw), abs=1e-12)
        assert layouts.scale_group(fmt) == int(group)
    assert layouts.BLOCK_BYTES["rocmfp4_dual"] == 18 and layouts.BLOCK_BYTES["rocmfp4_fast"] == 17
    assert layouts.canonical_bytes("nvfp4", 2048, 2048) == 2048 * (1024 + 128)


def test_layout_roundtrip():
    rng = np.random.default_rng(3)
    for fmt in ("rocmfp4_dual", "rocmfp4_fast"):
        blocks = rng.integers(0, 256, size=(3, 4, layouts.BLOCK_BYTES[fmt]), dtype=np.uint8)
        codes, sc = layouts.rocm_split(fmt, blocks)
        assert codes.shape == (3, 128)
        assert np.array_equal(layouts.rocm_join(fmt, codes, sc), blocks)
    wq = rng.integers(0, 256, size=(5, 8), dtype=np.uint8)
    assert np.array_equal(layouts.nvfp4_join(layouts.nvfp4_split(wq)), wq)
    blocks = rng.integers(0, 256, size=(3, 4, 18), dtype=np.uint8)
    codes, d = layouts.q4_0_split(blocks)
    assert codes.shape == (3, 128) and d.shape == (3, 4)
    assert np.array_equal(layouts.q4_0_join(codes, d), blocks)


def test_q4_0_grid_is_uniform_integer_steps():
    # comparison table, stock Q4_0: uniform integer steps; 16 codes -> the 16 consecutive integers -8..7
    lv = formats.q4_0_value(np.arange(16))
    assert lv.tolist() == list(range(-8, 8))
    assert np.all(np.diff(lv) == 1.0)


def _fp16_closed_form(b: int) -> float:
    s, e, m = b >> 15, (b >> 10) & 31, b & 1023
    if e == 31:
        return float("nan") if m else (-1) ** s * float("inf")
    mag = m * 2.0 ** -24 if e == 0 else (1024 + m) * 2.0 ** (e - 25)
    return -mag if s else mag


def test_fp16_codec_all_patterns():
    # decode: every pattern against the IEEE binary16 closed form and against torch's decoder
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = formats.fp16_value(bits)
    want = np.array([_fp16_closed_form(int(b)) for b in bits])
    assert np.array_equal(v, want, equal_nan=True)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.float16).to(torch.float64).numpy()
    assert np.array_equal(v, t, equal_nan=True)
    # encode: nearest finite value, ties to the even pattern, on values between and at the grid points
    pos = np.sort(want[np.isfinite(want) & (want >= 0)])
    pos = np.unique(pos)
    rng = np.random.default_rng(4)
    i = rng.integers(0, len(pos) - 1, 3000)
    lo, hi = pos[i], pos[i + 1]
    probes = np.concatenate([lo, (lo + hi) / 2, lo + (hi - lo) * rng.random(3000)])
    got = formats.fp16_value(formats.fp16_encode_rne(probes))
    for p, gv in zip(probes, got):
        j = np.searchsorted(pos, p)
        cands = [c for c in (pos[max(j - 1, 0)], pos[min(j, len(pos) - 1)])]
        best = min(cands, key=lambda c: (abs(c - p), int(formats.fp16_encode_rne(c)) & 1))
        assert gv == best, (p, gv, best)


def test_widget_q4_0_shared_scale_displays_as_page():
    # section 02's lab shows a Q4_0 shared scale of 1.025 beside ROCmFP4 half scales 0.813 / 0.094;
    # under the signed abs-max rule that is an outlier of magnitude 8.2 (8.2 / 8 = 1.025), and its
    # FP16 scale prints as 1.025 to three decimals
    d16 = formats.fp16_value(formats.fp16_encode_rne(8.2 / 8.0))
    assert f"{abs(float(d16)):.3f}" == "1.025"
