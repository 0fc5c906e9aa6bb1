"""Pins of the oracle's dequantisation and product (CPU)."""
import math

import numpy as np

import synth
from oracle import layouts, pack, ref
from tests import golden_io


def _hand():
    return golden_io.read("hand_packed.txt")


def test_dequant_dual_hand_packed():
    g = _hand()
    qs = golden_io.hex_bytes(g["qs"])
    block = np.array(golden_io.hex_bytes(g["dual_scales"]) + qs, dtype=np.uint8).reshape(1, 1, 18)
    w = ref.dequant("rocmfp4_dual", (block, np.float32(1)))
    assert w.tolist() == [golden_io.floats(g["dual_values"])]


def test_dequant_fast_hand_packed():
    g = _hand()
    qs = golden_io.hex_bytes(g["qs"])
    block = np.array(golden_io.hex_bytes(g["fast_scale"]) + qs, dtype=np.uint8).reshape(1, 1, 17)
    w = ref.dequant("rocmfp4_fast", (block, np.float32(1)))
    assert w.tolist() == [golden_io.floats(g["fast_values"])]


def test_dequant_nvfp4_hand_packed():
    g = _hand()
    wq = np.array(golden_io.hex_bytes(g["qs"]), dtype=np.uint8).reshape(1, 16)
    ws = np.array(golden_io.hex_bytes(g["nvfp4_scales"]), dtype=np.uint8).reshape(1, 2)
    w = ref.dequant("nvfp4", (wq, ws, np.float32(g["nvfp4_g"][0])))
    want = golden_io.floats(g["nvfp4_values"])
    assert w.tolist() == [want]
    assert np.array_equal(np.signbit(w[0]), np.signbit(np.array(want)))


def test_dequant_q4_0_hand_packed():
    g = _hand()
    qs = golden_io.hex_bytes(g["qs"])
    block = np.array(golden_io.hex_bytes(g["q4_0_scale_bytes"]) + qs, dtype=np.uint8).reshape(1, 1, 18)
    w = ref.dequant("q4_0", (block, np.float32(1)))
    assert w.tolist() == [golden_io.floats(g["q4_0_values"])]


def test_dequant_f32_is_single_rounding_of_exact_product():
    # e2m1 * e4m3 has <= 6 significant bits, so fl32(fl32(level*scale)*g) is the RN of the exact value,
    # while fl32(level*fl32(scale*g)) is not in general. The oracle rounds the exact product once.
    rng = np.random.default_rng(11)
    wq = rng.integers(0, 256, size=(64, 64), dtype=np.uint8)
    ws = rng.integers(0, 0x7F, size=(64, 8), dtype=np.uint8)
    g = np.float32(0.1234567)
    w32 = ref.dequant_f32("nvfp4", (wq, ws, g))
    codes = layouts.nvfp4_split(wq)
    from oracle import formats
    lv = formats.e2m1_value(codes).astype(np.float32)
    sc = np.repeat(formats.e4m3_value(ws).astype(np.float32), 16, axis=1)
    two_step = (lv * sc) * g                     # float32 ops: exact product then one rounding
    assert np.array_equal(w32, two_step.astype(np.float32))


def test_matmul_matches_fsum():
    rng = np.random.default_rng(5)
    w = rng.standard_normal((7, 48))
    x_bits = synth.activations(3, 48, cfg=99)
    x = ref.bf16_bits_to_f64(x_bits)
    y = ref.matmul(x_bits, w)
    for m in range(3):
        for n in range(7):
            assert abs(y[m, n] - math.fsum(x[m, k] * w[n, k] for k in range(48))) <= 1e-12 * (
                math.fsum(abs(x[m, k] * w[n, k]) for k in range(48)) + 1e-300)
    b = ref.bound(x_bits, w)
    assert np.allclose(b, np.abs(x) @ np.abs(w).T, rtol=0, atol=0)


def test_one_hot_x_returns_weight_columns():
    w = np.arange(12.0).reshape(3, 4)
    for k in range(4):
        x_bits = np.zeros((1, 4), np.uint16)
        x_bits[0, k] = 0x3F80                      # bf16 1.0
        assert np.array_equal(ref.matmul(x_bits, w)[0], w[:, k])


def test_all_equal_level_unit_scale_gives_level_times_sum_x():
    # every code = level 3 (code 3), every UE4M3 scale 0x38 = 1.0  ->  y = 3 * sum(x)
    n, k = 4, 64
    qs = np.full((n, k // 32, 16), 0x33, np.uint8)
    blocks = np.concatenate([np.full((n, k // 32, 1), 0x38, np.uint8), qs], axis=2)
    x_bits = synth.activations(2, k, cfg=98)
    y = ref.matmul(x_bits, ref.dequant("rocmfp4_fast", (blocks, np.float32(1))))
    sx = ref.bf16_bits_to_f64(x_bits).sum(axis=1)
    assert np.allclose(y, 3.0 * sx[:, None], rtol=1e-15, atol=1e-12)


def test_bf16_conversion_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0001, 0x7F7F, 0x4120, 0x0000, 0x8000], np.uint16)
    v = ref.bf16_bits_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -1.0 and v[2] == 2.0 ** -133 and v[4] == 10.0
    assert v[3] == (2 - 2.0 ** -7) * 2.0 ** 127


def test_tolerance_check():
    y_ref = np.array([[1.0, -2.0]])
    b = np.array([[10.0, 10.0]])
    ok, worst = ref.check(np.array([[1.0 + 0.019, -2.0]]), y_ref, b)
    assert ok and worst < 1
    ok, _ = ref.check(np.array([[1.0 + 0.021, -2.0]]), y_ref, b)
    assert not ok
    ok, _ = ref.check(np.array([[np.nan, -2.0]]), y_ref, b)
    assert not ok


def test_packed_roundtrip_error_small():
    # not a pin of exactness, a sanity bound: 4-bit block-scaled RTN / MSE fits are within ~15 % RMS
    w = synth.weights(64, 256, dist="t", nu=5, cfg=97)
    for fmt in ("nvfp4", "rocmfp4_dual", "rocmfp4_fast"):
        w64 = ref.dequant(fmt, pack.pack(fmt, w))
        rel = np.sqrt(np.mean((w64 - w) ** 2)) / np.sqrt(np.mean(w.astype(np.float64) ** 2))
        assert rel < 0.15, (fmt, rel)
