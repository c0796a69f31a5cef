"""Pins for oracle.quant: round-trip invariants, error bounds, spec rules.

A plausible mistake in a quantizer (wrong divisor, wrong zero-point sign,
unstored scale, wrong shared-exponent rule, wrong clamp) breaks one of these.
"""

import numpy as np
import torch

import synth
from oracle import codecs, quant, ref


def _f16_scales(r, shape):
    # fp16 scales of the size quantized N(0, 0.02) weights produce
    return codecs.f32_to_f16_bits(r.uniform(1e-3, 1e-2, shape).astype(np.float32))


def test_int4_sym_roundtrip_recovers_codes():
    r = np.random.default_rng(10)
    n, k, g = 8, 512, 128
    q = r.integers(-7, 8, size=(n, k))
    q[:, ::g] = 7 * np.where(r.random((n, k // g)) < 0.5, 1, -1)  # each group reaches |7|
    s = _f16_scales(r, (n, k // g))
    w = ref.dequant_int4_sym(q, s).astype(np.float32)
    q2, s2 = quant.quantize_int4_sym(w, g)
    assert np.array_equal(s2, s)
    assert np.array_equal(q2, q)


def test_int4_sym_error_bound_and_range():
    w = synth.weights_f32(64, 1024, workload_id=1, salt=7)
    q, s = quant.quantize_int4_sym(w)
    assert q.min() >= -8 and q.max() <= 7
    deq = ref.dequant_int4_sym(q, s)
    sc = np.repeat(codecs.f16_bits_to_f64(s), 128, axis=1)
    assert np.all(np.abs(deq - w) <= sc * 0.5 * (1 + 1e-3))
    # the scale is amax/7 rounded to fp16 (amax/8 would leave |q| <= 7 unused)
    amax = np.abs(w.reshape(64, 8, 128)).max(axis=2)
    assert np.allclose(codecs.f16_bits_to_f64(s), amax / 7, rtol=2 ** -10)


def test_uint4_asym_roundtrip_and_bounds():
    r = np.random.default_rng(11)
    n, k, g = 8, 256, 128
    q = r.integers(0, 16, size=(n, k))
    q[:, 0::g] = 0
    q[:, 1::g] = 15
    z = r.integers(0, 16, size=(n, k // g)).astype(np.uint8)
    s = _f16_scales(r, (n, k // g))
    w = ref.dequant_uint4_asym(q, s, z).astype(np.float32)
    q2, s2, z2 = quant.quantize_uint4_asym(w, g)
    # the range is 15 s exactly, so the stored scale comes back ...
    assert np.array_equal(s2, s)
    # ... and so do zero point and codes
    assert np.array_equal(z2, z)
    assert np.array_equal(q2, q)


def test_uint4_asym_error_bound():
    w = synth.weights_f32(32, 1024, workload_id=0, salt=3)
    q, s, z = quant.quantize_uint4_asym(w)
    assert q.min() >= 0 and q.max() <= 15 and z.max() <= 15
    deq = ref.dequant_uint4_asym(q, s, z)
    sc = np.repeat(codecs.f16_bits_to_f64(s), 128, axis=1)
    err = np.abs(deq - w)
    inner = (q > 0) & (q < 15)
    assert np.all(err[inner] <= sc[inner] * 0.5 * (1 + 1e-3))
    assert np.all(err <= sc * 1.5)
    # the zero point sits where real zero falls: deq of code z is 0
    assert np.all(np.abs(ref.dequant_uint4_asym(np.repeat(z.astype(np.int64), 128, axis=1), s, z)) == 0)


def test_int8_per_channel():
    w = synth.weights_f32(16, 512, workload_id=2, salt=1)
    q, s = quant.quantize_int8_per_channel(w)
    assert np.abs(q).max() == 127
    assert np.all(np.abs(q * s[:, None].astype(np.float64) - w) <= s[:, None] * 0.5 * (1 + 1e-6))
    # round trip on exact grid values
    q2, s2 = quant.quantize_int8_per_channel((q * s[:, None]).astype(np.float32))
    assert np.array_equal(q2, q)


def test_mxfp4_shared_exponent_rule_and_error():
    w = synth.weights_f32(16, 1024, workload_id=3, salt=2)
    codes, e = quant.quantize_mxfp4(w)
    x = e.astype(np.int64) - 127
    amax = np.abs(w.reshape(16, 32, 32)).max(axis=2).astype(np.float64)
    # OCP MX: X = floor(log2(amax)) - 2, i.e. amax / 2**X lies in [4, 8)
    ratio = amax / np.ldexp(1.0, x)
    assert np.all((ratio >= 4) & (ratio < 8))
    deq = ref.dequant_mxfp4(codes, e)
    scale = np.repeat(np.ldexp(1.0, x), 32, axis=1)
    y = w / scale
    # E2M1 spacing: 0.5 below 2, 1 in [2,4), 2 in [4,6]; values above 6 saturate
    half_gap = np.where(np.abs(y) < 2, 0.25, np.where(np.abs(y) < 4, 0.5, 1.0))
    sat = np.abs(y) > 6
    assert np.all(np.abs(deq - w)[~sat] <= (half_gap * scale)[~sat] * (1 + 1e-9))
    assert np.all(np.abs(deq[sat]) == 6 * scale[sat])


def test_mxfp4_zero_block_and_roundtrip():
    r = np.random.default_rng(12)
    codes = r.integers(0, 16, size=(4, 64)).astype(np.uint8)
    codes[:, 0::32] = 0x7  # each block reaches 6 -> exponent rule recovers X
    e = r.integers(110, 130, size=(4, 2)).astype(np.uint8)
    w = ref.dequant_mxfp4(codes, e).astype(np.float32)
    c2, e2 = quant.quantize_mxfp4(w)
    assert np.array_equal(e2, e)
    # -0 and +0 decode alike; compare values
    assert np.array_equal(codecs.decode_e2m1(c2), codecs.decode_e2m1(codes))
    z = np.zeros((2, 32), np.float32)
    cz, ez = quant.quantize_mxfp4(z)
    assert np.all(cz == 0) and np.all(ez == 0)


def test_act_int8_properties():
    a = synth.activations_bf16_bits(64, 512, workload_id=2, salt=4)
    a[3] = 0  # an all-zero row
    qa, sa = quant.quantize_act_int8(a)
    x = codecs.bf16_bits_to_f64(a)
    assert qa.dtype == np.int8 and np.abs(qa.astype(int)).max() <= 127
    assert sa[3] == 1.0 and np.all(qa[3] == 0)
    rows = [i for i in range(64) if i != 3]
    amax = np.abs(x[rows]).max(axis=1)
    assert np.allclose(sa[rows], amax / 127, rtol=2 ** -23)
    # the largest element maps to +-127
    am = np.abs(x[rows]).argmax(axis=1)
    assert np.all(np.abs(qa[rows, am].astype(int)) == 127)
    err = np.abs(qa[rows] * sa[rows, None].astype(np.float64) - x[rows])
    assert np.all(err <= sa[rows, None] * 0.5 * (1 + 1e-5))


def test_act_fp8_codes_match_torch_cast():
    a = synth.activations_bf16_bits(16, 1024, workload_id=3, salt=5)
    a[2, 128:256] = 0  # an all-zero group
    codes, sa = quant.quantize_act_fp8(a)
    assert sa[2, 1] == 1.0 and np.all(codes[2, 128:256] == 0)
    x = codecs.bf16_bits_to_f64(a).astype(np.float32).reshape(16, 8, 128)
    amax = np.abs(x).max(axis=2)
    nz = amax > 0
    inv = np.float32(448.0) / np.where(nz, amax, np.float32(1))
    v = np.clip(x * inv[:, :, None], -448, 448).astype(np.float32)
    ref_codes = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ref_codes = np.where(nz[:, :, None], ref_codes, 0).reshape(16, 1024)
    assert np.array_equal(codes, ref_codes)
    # largest element of each group maps to +-448 exactly
    dec = codecs.decode_e4m3(codes).reshape(16, 8, 128)
    assert np.all(np.abs(dec).max(axis=2)[nz] == 448.0)


def test_act_mxfp4_is_the_block_rule_on_each_row():
    # rows of exactly representable values: every block reaches +-6 * 2**X,
    # so the shared exponent is X and the codes round-trip exactly
    r = np.random.default_rng(41)
    m, k = 3, 96
    codes = r.integers(0, 16, size=(m, k)).astype(np.uint8)
    codes[:, 5::32] = 0xF  # -6 in every block
    e = r.integers(118, 134, size=(m, k // 32)).astype(np.uint8)
    x = ref.dequant_mxfp4(codes, e)
    bits = codecs.f32_to_bf16_bits(x.astype(np.float32))
    assert np.array_equal(codecs.bf16_bits_to_f64(bits), x)  # exact in bf16
    c2, e2 = quant.quantize_act_mxfp4(bits)
    assert np.array_equal(e2, e)
    assert np.array_equal(codecs.decode_e2m1(c2), codecs.decode_e2m1(codes))
    # hand block: amax 1.0 -> X = -2 (scale 1/4); 0.3/0.25 = 1.2 -> 1.0 (code 2);
    # 0.0625/0.25 = 0.25 -> tie between 0 and 0.5 -> even -> 0; -0.1875/0.25 =
    # -0.75 -> tie between 0.5 and 1.0 -> even -> -1.0 (code 0xA); 1.0 -> 4 (code 6)
    row = np.zeros((1, 32), np.float32)
    row[0, :4] = [0.3, 0.0625, -0.1875, 1.0]
    c3, e3 = quant.quantize_act_mxfp4(codecs.f32_to_bf16_bits(row))
    assert e3[0, 0] == 125
    assert list(c3[0, :4]) == [2, 0, 0xA, 6]


def test_uint2_asym_roundtrip_bounds_and_packing():
    # grid values (q - z) * s with every group reaching codes 0 and 3 come
    # back exactly: scale, zero point and codes
    r = np.random.default_rng(13)
    n, k, g = 6, 256, 128
    q = r.integers(0, 4, size=(n, k))
    q[:, 0::g] = 0
    q[:, 1::g] = 3
    z = r.integers(0, 4, size=(n, k // g)).astype(np.uint8)
    s = _f16_scales(r, (n, k // g))
    w = ref.dequant_uint2_asym(q, s, z).astype(np.float32)
    q2, s2, z2 = quant.quantize_uint2_asym(w, g)
    assert np.array_equal(s2, s) and np.array_equal(z2, z) and np.array_equal(q2, q)
    # error bound on N(0, 0.02) weights: inside the code range within s/2,
    # and the zero point's code dequantizes to 0
    w = synth.weights_f32(16, 512, workload_id=1, salt=9)
    q, s, z = quant.quantize_uint2_asym(w)
    assert q.min() >= 0 and q.max() <= 3 and z.max() <= 3
    deq = ref.dequant_uint2_asym(q, s, z)
    sc = np.repeat(codecs.f16_bits_to_f64(s), 128, axis=1)
    inner = (q > 0) & (q < 3)
    assert np.all(np.abs(deq - w)[inner] <= sc[inner] * 0.5 * (1 + 1e-3))
    assert np.all(ref.dequant_uint2_asym(np.repeat(z.astype(np.int64), 128, axis=1), s, z) == 0)
    # the scale is the group's range over 3 rounded to fp16
    wg = w.reshape(16, 4, 128)
    assert np.allclose(codecs.f16_bits_to_f64(s), (wg.max(axis=2) - wg.min(axis=2)) / 3, rtol=2 ** -10)
    # 2-bit packing: element k in byte k/4 at bits 2 (k % 4); hand byte and round trip
    assert list(codecs.pack_crumbs(np.array([[1, 2, 3, 0]]))[0]) == [1 | (2 << 2) | (3 << 4)]
    codes = r.integers(0, 4, size=(3, 64)).astype(np.uint8)
    assert np.array_equal(codecs.unpack_crumbs(codecs.pack_crumbs(codes)), codes)
