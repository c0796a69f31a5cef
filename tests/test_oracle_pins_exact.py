"""Pins for the parts of the oracle that every parity test leans on:

* ``metrics.rel_frob`` against hand-computed values (a wrong norm, a missing
  square root or the wrong denominator fails here);
* the activation quantizers' stored scales and codes against the binary32
  steps the readings fix, evaluated here in exact rational arithmetic
  (``fractions.Fraction``) with a correctly rounded binary32 / E4M3 rounding
  written from the IEEE 754 and OCP 8-bit definitions, not with numpy's
  float32 or the oracle's codecs.

The quantizer readings (kinachrichten, "Warum quantisierte Kernel wichtig
sind", names per-token int8 and per-group fp8 activations without a recipe):
int8 per row, ``inv = f32(127 / amax)``, ``q = clamp(rne(f32(x * inv)), ±127)``,
stored ``sa = f32(amax / 127)``; fp8 E4M3 per (row, 128-group), ``inv =
f32(448 / amax)``, ``q = e4m3_rne(clamp(f32(x * inv), ±448))``, stored ``sa =
f32(amax / 448)``. The hand rows below are chosen so that the other plausible
reading, dividing by the stored scale (``x / sa``), gives a different code for
at least one element; the test asserts that too, so it discriminates.
"""

import math
from fractions import Fraction as Fr

import numpy as np

from oracle import codecs, metrics, quant


# ---------------------------------------------------------------- rel_frob

def test_rel_frob_hand_values():
    # ||[[0,0],[0,-1]]||_F / ||[[1,0],[0,2]]||_F = 1 / sqrt(5)
    y = np.array([[1.0, 0.0], [0.0, 1.0]])
    r = np.array([[1.0, 0.0], [0.0, 2.0]])
    assert abs(metrics.rel_frob(y, r) - 1 / math.sqrt(5)) < 1e-15
    # a 3-4-5 difference against a norm-10 reference: 5 / 10 (an L1 norm
    # would give 0.7 / 0.6..., a max norm 0.4 / 0.8, a squared norm 0.25)
    y = np.array([3.0, 4.0, 6.0, 8.0])
    r = np.array([0.0, 0.0, 6.0, 8.0])
    assert metrics.rel_frob(y, r) == 0.5
    # symmetric in sign, scale invariant, zero for equal inputs
    assert metrics.rel_frob(-y, -r) == 0.5
    assert metrics.rel_frob(4 * y, 4 * r) == 0.5
    assert metrics.rel_frob(r, r) == 0.0
    # the reference is the denominator, not the result
    assert abs(metrics.rel_frob(np.array([2.0]), np.array([1.0])) - 1.0) < 1e-15
    assert abs(metrics.rel_frob(np.array([1.0]), np.array([2.0])) - 0.5) < 1e-15
    # a zero reference falls back to the absolute norm
    assert metrics.rel_frob(np.array([3.0, 4.0]), np.zeros(2)) == 5.0
    # float32 inputs are compared in float64 (no float32 rounding of the
    # difference: 1 + 2^-20 and 1 differ by exactly 2^-20)
    a = np.array([1 + 2 ** -20], dtype=np.float32)
    b = np.array([1.0], dtype=np.float32)
    assert metrics.rel_frob(a, b) == 2 ** -20


# --------------------------------------- exact binary32 / E4M3 rounding

def _rne_int(v):
    """Round a Fraction to the nearest integer, ties to even."""
    f = math.floor(v)
    d = v - f
    if d > Fr(1, 2) or (d == Fr(1, 2) and f % 2 == 1):
        return f + 1
    return f


def f32_rne(v):
    """Correctly rounded binary32 value of a rational (IEEE 754 RNE; no
    overflow handling needed for the magnitudes used here)."""
    if v == 0:
        return Fr(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fr(2) ** e > a:
        e -= 1
    while Fr(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                      # subnormals share the least exponent
    ulp = Fr(2) ** (e - 23)
    return sign * _rne_int(a / ulp) * ulp


def _e4m3_values():
    """Every finite non-negative OCP E4M3 ("fn") value with its code: exponent
    bias 7, 3 mantissa bits, subnormals 2^-6 * m/8, and 0x7F the NaN."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        v = Fr(m, 8) * Fr(2) ** -6 if e == 0 else (1 + Fr(m, 8)) * Fr(2) ** (e - 7)
        vals.append((v, code))
    return vals


E4M3 = _e4m3_values()


def e4m3_rne_code(v):
    """OCP E4M3 code of a rational |v| <= 448, rounded to nearest, ties to the
    even code (even mantissa)."""
    a = abs(v)
    best = min(E4M3, key=lambda t: (abs(t[0] - a), t[1] & 1))
    code = best[1]
    return code | (0x80 if v < 0 and code != 0 else 0)


def _bits32(fr):
    return int(np.array([float(fr)], dtype=np.float32).view(np.uint32)[0])


def _bf16_row(values):
    """bf16 bit patterns of values that are exact in bf16 (checked)."""
    out = codecs.f32_to_bf16_bits(np.array(values, dtype=np.float32))
    assert np.array_equal(codecs.bf16_bits_to_f64(out), np.array(values, dtype=np.float64))
    return out


# ----------------------------------------------------- int8 activations

def _int8_expected(row):
    xs = [Fr(float(v)) for v in row]
    amax = max(abs(x) for x in xs)
    if amax == 0:
        return [0] * len(xs), Fr(1), [0] * len(xs)
    inv = f32_rne(Fr(127) / amax)
    sa = f32_rne(amax / 127)
    q_mul = [max(-127, min(127, _rne_int(f32_rne(x * inv)))) for x in xs]
    q_div = [max(-127, min(127, _rne_int(f32_rne(x / sa)))) for x in xs]
    return q_mul, sa, q_div


# (amax, x) pairs of bf16 values where f32(x * f32(127/amax)) and
# f32(x / f32(amax/127)) fall on opposite sides of a .5 tie (x = amax/2 is
# the tie 63.5 itself), found by a scan over bf16 values; the test
# recomputes both readings exactly and checks that they differ
INT8_SPLIT = [(1.1484375, 0.57421875), (1.2578125, 0.62890625), (2.265625, 1.1328125),
              (3.359375, 1.6796875), (6.21875, 3.109375)]


def test_act_int8_scale_and_codes_exact():
    rows = []
    for amax, x in INT8_SPLIT:
        rows.append([amax, -x, x, 0.0, -amax, amax / 4, 0.0078125])
    rows.append([0.0029296875, -0.0029296875, 0.00146484375, 0.0, 1e-30, 0.0, 0.0])
    rows.append([0.0] * 7)  # an all-zero row: sa = 1, codes 0
    rows = [[float(codecs.bf16_bits_to_f64(codecs.f32_to_bf16_bits(np.array([v], np.float32)))[0])
             for v in r] for r in rows]
    bits = np.stack([_bf16_row(r) for r in rows])
    qa, sa = quant.quantize_act_int8(bits)
    separated = 0
    for i, r in enumerate(rows):
        q_mul, s_exp, q_div = _int8_expected(r)
        assert _bits32(s_exp) == int(sa[i:i + 1].view(np.uint32)[0]), (i, r)
        assert list(qa[i].astype(int)) == q_mul, (i, r)
        separated += q_mul != q_div
    # the rows separate the reading from dividing by the stored scale
    assert separated >= len(INT8_SPLIT)


# ------------------------------------------------------ fp8 activations

def _fp8_expected(group):
    xs = [Fr(float(v)) for v in group]
    amax = max(abs(x) for x in xs)
    if amax == 0:
        return [0] * len(xs), Fr(1), [0] * len(xs)
    inv = f32_rne(Fr(448) / amax)
    sa = f32_rne(amax / 448)

    def enc(v):
        return e4m3_rne_code(max(Fr(-448), min(Fr(448), v)))
    q_mul = [enc(f32_rne(x * inv)) for x in xs]
    q_div = [enc(f32_rne(x / sa)) for x in xs]
    return q_mul, sa, q_div


# (amax, x) pairs where the two readings round f32(x * inv) and f32(x / sa)
# to different E4M3 codes (ties in the subnormal range), found by a scan
FP8_SPLIT = [(0.5, 7.62939453125e-06), (0.6484375, 9.894371032714844e-06),
             (0.7109375, 2.014636993408203e-05), (0.765625, 2.1696090698242188e-05)]


def test_act_fp8_scale_and_codes_exact():
    g = 128
    rng = np.random.default_rng(7)
    groups = []
    for amax, x in FP8_SPLIT + [(3.0, 1.5), (200.0, 0.25), (0.0029296875, 1e-6)]:
        vals = [amax, -amax, x, -x]
        # bf16 values spread over the group's range
        raw = rng.uniform(-amax, amax, g - 4).astype(np.float32)
        vals += list(codecs.bf16_bits_to_f64(codecs.f32_to_bf16_bits(raw)))
        vals = [min(max(v, -amax), amax) for v in vals]
        vals = [float(codecs.bf16_bits_to_f64(codecs.f32_to_bf16_bits(np.array([v], np.float32)))[0])
                for v in vals]
        groups.append(vals)
    groups.append([0.0] * g)  # an all-zero group: scale 1, codes 0
    row = sum(groups, [])
    bits = _bf16_row(row)[None, :]
    codes, sa = quant.quantize_act_fp8(bits, group=g)
    separated = 0
    for j, grp in enumerate(groups):
        q_mul, s_exp, q_div = _fp8_expected(grp)
        assert _bits32(s_exp) == int(sa[0, j:j + 1].view(np.uint32)[0]), j
        got = [int(c) for c in codes[0, j * g:(j + 1) * g]]
        norm = [c if c & 0x7F else 0 for c in got]  # -0 and +0 alike
        assert norm == q_mul, j
        separated += q_mul != q_div
    assert separated >= len(FP8_SPLIT), "the hand groups must separate the two readings"


def test_exact_helpers_against_known_values():
    # the helpers themselves: binary32 RNE of 1/3, 127/3 and a tie; E4M3 ends
    assert _bits32(f32_rne(Fr(1, 3))) == 0x3EAAAAAB
    assert float(f32_rne(Fr(1) + Fr(1, 2 ** 24))) == 1.0          # tie -> even
    assert float(f32_rne(Fr(1) + Fr(3, 2 ** 24))) == 1 + 2 ** -22  # tie -> even (up)
    assert e4m3_rne_code(Fr(448)) == 0x7E
    assert e4m3_rne_code(Fr(-448)) == 0xFE
    assert e4m3_rne_code(Fr(1)) == 0x38
    assert e4m3_rne_code(Fr(2) ** -9) == 0x01                      # least subnormal
    assert e4m3_rne_code(Fr(2) ** -10) == 0x00                     # tie -> even (0)
    assert e4m3_rne_code(Fr(3) * Fr(2) ** -10) == 0x02             # tie -> even (2)
    assert e4m3_rne_code(Fr(17, 16)) == 0x38                       # 1.0625: tie -> 1.0
    assert e4m3_rne_code(Fr(19, 16)) == 0x3A                       # 1.1875: tie -> 1.25
