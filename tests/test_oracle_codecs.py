"""Pins for oracle.codecs against the specifications and independent library casts.

OCP MX v1.0 (E2M1, E8M0), OCP OFP8 (E4M3), IEEE 754 (bf16/fp16 RNE). torch's
float8_e4m3fn / float8_e8m0fnu / bfloat16 casts are independent
implementations of the same definitions and serve as second opinions.
"""

import numpy as np
import pytest
import torch

from oracle import codecs


def test_int4_nibbles_hand_cases():
    # two's complement: 0x8 is the most negative value, 0xF is -1
    assert codecs.decode_int4([0x0, 0x7, 0x8, 0xF]).tolist() == [0, 7, -8, -1]
    assert codecs.encode_int4([-8, -1, 0, 7]).tolist() == [8, 15, 0, 7]
    # element 0 in the low nibble, element 1 in the high nibble
    assert codecs.pack_nibbles(np.array([1, 2, 15, 0])).tolist() == [0x21, 0x0F]
    assert codecs.unpack_nibbles(np.array([0x21, 0x0F], np.uint8)).tolist() == [1, 2, 15, 0]


def test_nibble_pack_roundtrip():
    r = np.random.default_rng(0)
    c = r.integers(0, 16, size=(5, 64))
    assert np.array_equal(codecs.unpack_nibbles(codecs.pack_nibbles(c)), c)


def test_e2m1_table_matches_spec():
    # OCP MX v1.0 FP4 E2M1 element values for codes 0..7; codes 8..15 negate them
    expect = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = codecs.decode_e2m1(np.arange(16))
    assert got[:8].tolist() == expect
    assert (-got[8:]).tolist() == expect
    assert np.signbit(got[8])  # code 0x8 is -0


def test_e2m1_encoder_brute_force():
    vals = codecs.decode_e2m1(np.arange(8))
    mids = (vals[1:] + vals[:-1]) / 2
    r = np.random.default_rng(1)
    xs = np.concatenate([vals, mids, -mids, r.uniform(-8, 8, 5000), [7.0, -100.0, 6.0, 1e9]])
    codes = codecs.encode_e2m1_rne_sat(xs)
    dec = codecs.decode_e2m1(codes)
    for x, c, d in zip(xs, codes, dec):
        target = np.clip(x, -6.0, 6.0)
        # brute force over all 16 codes with the same sign
        cand = [cc for cc in range(16) if (cc >> 3) == int(np.signbit(x))]
        dist = [abs(codecs.decode_e2m1(cc) - target) for cc in cand]
        best = min(dist)
        ties = [cc for cc, dd in zip(cand, dist) if dd == best]
        assert abs(d - target) == best, (x, c)
        if len(ties) > 1:
            assert (int(c) & 1) == 0, (x, c, ties)  # ties to even mantissa


def test_e8m0_matches_torch():
    codes = np.arange(255, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(codecs.decode_e8m0(codes), ref)
    assert codecs.decode_e8m0([127, 128, 126]).tolist() == [1.0, 2.0, 0.5]
    assert np.isnan(codecs.decode_e8m0([255]))[0]


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = codecs.decode_e4m3(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    # spec landmarks: max normal 448, min subnormal 2**-9, min normal 2**-6
    assert codecs.decode_e4m3([0x7E, 0x01, 0x08, 0x38]).tolist() == [448.0, 2.0 ** -9, 2.0 ** -6, 1.0]


def test_e4m3_encode_matches_torch():
    r = np.random.default_rng(2)
    table = codecs.decode_e4m3(np.arange(0x7F))
    mids = (table[1:] + table[:-1]) / 2
    xs = np.concatenate([table, -table, mids, -mids, r.uniform(-448, 448, 20000),
                         r.standard_normal(20000) * 1e-2]).astype(np.float32)
    got = codecs.encode_e4m3_rne(xs)
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_bf16_rne_matches_torch():
    r = np.random.default_rng(3)
    base = r.standard_normal(20000).astype(np.float32)
    u = base.view(np.uint32)
    ties = ((u & 0xFFFF0000) | 0x8000).view(np.float32)  # exact halfway cases
    xs = np.concatenate([base, ties, np.float32([0.0, -0.0, 3.0e38, 1e-40])])
    got = codecs.f32_to_bf16_bits(xs)
    ref = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    assert np.array_equal(codecs.bf16_bits_to_f64(got),
                          torch.from_numpy(xs).to(torch.bfloat16).to(torch.float64).numpy())


def test_f16_roundtrip_exact():
    bits = np.arange(0, 0x7C00, 7, dtype=np.uint16)  # finite positive halves
    v = codecs.f16_bits_to_f64(bits)
    assert np.array_equal(codecs.f32_to_f16_bits(v.astype(np.float32)), bits)
