"""Pins of the oracle's NVFP4 pieces (E2M1 elements, E4M3 scales per 16 K,
one binary32 scale per tensor) against values fixed by the formats
themselves, exact rational brute force and special cases that reduce to
other, separately pinned oracle functions."""

from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import codecs, quant, ref

# E2M1 magnitudes by hand (OCP MX v1.0 table) and E4M3 from its bit fields
_E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def _e2m1_exact(c):
    v = _E2M1[c & 7]
    return -v if c & 8 else v


def _e4m3_exact(b):
    e, m = (b >> 3) & 15, b & 7
    v = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * (Fraction(2) ** (e - 7))
    return -v if b & 0x80 else v


def test_dequant_hand_values():
    # code 7 (+6) x scale 0x38 (1.0) x ts 0.5 = 3; code 0xB (-1.5) x 0x3C (1.5) = -2.25;
    # code 2 (+1) x subnormal 0x01 (2^-9) = 2^-9; code 0x7 x 0x7E (448) = 2688
    codes = np.array([[7] * 16 + [0xB] * 16 + [2] * 16 + [7] * 16], np.uint8)
    sc = np.array([[0x38, 0x3C, 0x01, 0x7E]], np.uint8)
    w = ref.dequant_nvfp4(codes, sc, np.float32(0.5))
    assert w[0, 0] == 3.0 and w[0, 16] == -2.25 * 0.5 and w[0, 32] == 2.0 ** -10 and w[0, 48] == 2688 * 0.5
    assert w.shape == (1, 64)


def test_nan_scale_rejected():
    with pytest.raises(AssertionError):
        ref.dequant_nvfp4(np.zeros((1, 16), np.uint8), np.array([[0x7F]], np.uint8), 1.0)


def test_gemm_brute_force_exact_rationals():
    # tiny GEMM over every E2M1 code and a spread of E4M3 scale codes, with
    # exact rational arithmetic; the float64 oracle is exact here (products
    # of <= 30 significant bits, sums of few terms far from 2^53 ulps)
    rng = np.random.default_rng(5)
    n, k, m = 3, 32, 2
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    codes[0, :16] = np.arange(16)
    sc = rng.choice([0x01, 0x07, 0x08, 0x30, 0x38, 0x3F, 0x55, 0x7E, 0xB8], (n, k // 16)).astype(np.uint8)
    ts = np.float32(2.0 ** -7 * 1.25)
    a_bits = synth.activations_bf16_bits(m, k, workload_id=0, salt=91)
    y = ref.gemm_nvfp4a16(a_bits, codes, sc, ts)
    a = codecs.bf16_bits_to_f64(a_bits)
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for kk in range(k):
                w = _e2m1_exact(int(codes[j, kk])) * _e4m3_exact(int(sc[j, kk // 16])) * Fraction(float(ts))
                acc += Fraction(float(a[i, kk])) * w
            assert abs(Fraction(float(y[i, j])) - acc) <= abs(acc) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)


def test_unit_scales_reduce_to_the_mxfp4_oracle():
    # E4M3 scale 1.0 (0x38) everywhere and ts = 1: the weights are the bare
    # E2M1 values, which the MXFP4 dequant gives with E8M0 code 127
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 16, (24, 256)).astype(np.uint8)
    w = ref.dequant_nvfp4(codes, np.full((24, 16), 0x38, np.uint8), np.float32(1.0))
    assert np.array_equal(w, ref.dequant_mxfp4(codes, np.full((24, 8), 127, np.uint8)))


def test_tensor_scale_power_of_two_is_exact():
    rng = np.random.default_rng(8)
    codes = rng.integers(0, 16, (8, 128)).astype(np.uint8)
    sc = rng.integers(0, 0x7F, (8, 8)).astype(np.uint8)
    a = synth.activations_bf16_bits(5, 128, workload_id=0, salt=92)
    y1 = ref.gemm_nvfp4a16(a, codes, sc, np.float32(0.375))
    y2 = ref.gemm_nvfp4a16(a, codes, sc, np.float32(0.75))
    assert np.array_equal(2.0 * y1, y2)


def test_one_hot_rows_give_the_dequantized_weights():
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 16, (6, 128)).astype(np.uint8)
    sc = rng.integers(0x20, 0x50, (6, 8)).astype(np.uint8)
    eye = codecs.f32_to_bf16_bits(np.eye(128, dtype=np.float32))
    y = ref.gemm_nvfp4a16(eye, codes, sc, np.float32(0.125))
    assert np.array_equal(y.T, ref.dequant_nvfp4(codes, sc, np.float32(0.125)))


def test_quantizer_scales_and_error_bound():
    w = synth.weights_f32(64, 512, workload_id=9, salt=1)
    codes, sc, ts = quant.quantize_nvfp4(w)
    amax = float(np.max(np.abs(w)))
    assert ts == np.float32(np.float32(amax) / np.float32(2688.0))
    # every block scale is the E4M3 rounding of amax_block / 6 / ts: within
    # half an E4M3 step (relative 1/16) of it
    blk = np.abs(w.reshape(64, 32, 16)).max(axis=2).astype(np.float64)
    target = blk / 6.0 / float(ts)
    got = codecs.decode_e4m3(sc)
    assert np.all(np.abs(got - target) <= target / 16 + 1e-300)
    # element error: at most half the E2M1 spacing at the element's magnitude
    # (spacing 0.5 below 2, 1 below 4, 2 up to 6), times the block's scale;
    # no element saturates because the block scale covers amax / 6
    deq = ref.dequant_nvfp4(codes, sc, ts).reshape(64, 32, 16)
    step = (got * float(ts))[:, :, None]
    x = w.reshape(64, 32, 16).astype(np.float64) / step
    half = np.where(np.abs(x) < 2, 0.25, np.where(np.abs(x) < 4, 0.5, 1.0))
    assert np.all(np.abs(deq / step - x) <= half * (1 + 1e-6) + 1e-12)


def test_quantizer_roundtrip_of_representable_weights():
    # weights built from codes, with one block at scale 448 holding a +-6 so
    # that the tensor scale is recovered exactly (a power of two), quantize
    # back to the same codes and scales
    rng = np.random.default_rng(11)
    n, k = 16, 256
    codes = rng.choice([c for c in range(16) if c != 8], (n, k)).astype(np.uint8)
    codes.reshape(n, k // 16, 16)[:, :, 0] = 7  # every block holds +6: amax = 6 * scale
    sc = rng.integers(0x08, 0x7E, (n, k // 16)).astype(np.uint8)
    sc[0, 0] = 0x7E
    ts = np.float32(2.0 ** -10)
    w = ref.dequant_nvfp4(codes, sc, ts).astype(np.float32)
    c2, s2, t2 = quant.quantize_nvfp4(w)
    assert t2 == ts and np.array_equal(s2, sc) and np.array_equal(c2, codes)


def test_quantizer_zero_tensor_and_zero_block():
    c, s, t = quant.quantize_nvfp4(np.zeros((2, 32), np.float32))
    assert t == np.float32(1.0) and not c.any() and not s.any()
    w = np.zeros((1, 32), np.float32)
    w[0, 16:] = 0.5
    c, s, t = quant.quantize_nvfp4(w)
    assert s[0, 0] == 0 and not c[0, :16].any()
    assert np.allclose(ref.dequant_nvfp4(c, s, t)[0, 16:], 0.5, rtol=1e-6, atol=0)
