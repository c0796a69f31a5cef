"""Exact decoders and round-to-nearest-even encoders for every storage type.

Test infrastructure (see the package docstring). Decoders return float64 (or
int64) values that are exact: every code of every type here is a dyadic
rational that binary64 holds without rounding.

Sources (external specifications, not the pages):
* OCP Microscaling Formats (MX) v1.0 -- FP4 E2M1 element (1 sign, 2 exponent,
  1 mantissa bit, bias 1, no inf/NaN, max 6) and the E8M0 shared scale
  (``2**(e-127)``, code 255 = NaN).
* OCP 8-bit Floating Point (OFP8) -- E4M3 (bias 7, no infinities, only
  S.1111.111 is NaN, max 448).
* IEEE 754 binary16 / binary32; bf16 = upper 16 bits of binary32.

The pages only say that 4-bit weights may be integer or floating point
(jetabc, section on what quantization is) and name MXFP4 (kinachrichten,
"Das Wichtigste in Kürze"); the bit layouts above are the specifications'.

Nibble packing (a reading, the pages give no layout): two 4-bit codes per byte,
element ``k`` in byte ``k // 2``, the even element in the low nibble.
"""

import numpy as np

# ---------------------------------------------------------------- nibbles


def unpack_nibbles(packed):
    """u8 [..., K/2] -> u8 codes [..., K]; even k in the low nibble."""
    packed = np.asarray(packed, dtype=np.uint8)
    lo = packed & 0x0F
    hi = packed >> 4
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def pack_nibbles(codes):
    """u8 codes [..., K] (0..15, K even) -> u8 [..., K/2]; inverse of unpack."""
    codes = np.asarray(codes)
    assert codes.shape[-1] % 2 == 0
    c = codes.astype(np.uint8) & 0x0F
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_crumbs(packed):
    """u8 [..., K/4] -> u8 2-bit codes [..., K]: element k in byte k/4, bits
    2 (k % 4) .. 2 (k % 4) + 1 (the lowest pair holds the first element)."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 4,), dtype=np.uint8)
    for j in range(4):
        out[..., j::4] = (packed >> (2 * j)) & 0x3
    return out


def pack_crumbs(codes):
    """u8 2-bit codes [..., K] (0..3, K a multiple of 4) -> u8 [..., K/4];
    inverse of unpack_crumbs."""
    codes = np.asarray(codes)
    assert codes.shape[-1] % 4 == 0
    c = codes.astype(np.uint8) & 0x3
    return (c[..., 0::4] | (c[..., 1::4] << 2) | (c[..., 2::4] << 4) | (c[..., 3::4] << 6)).astype(np.uint8)


def decode_int4(codes):
    """Two's-complement 4-bit code (0..15) -> integer in [-8, 7]."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    return np.where(c >= 8, c - 16, c)


def encode_int4(values):
    """Integer in [-8, 7] -> its two's-complement nibble (0..15)."""
    v = np.asarray(values).astype(np.int64)
    assert np.all((v >= -8) & (v <= 7))
    return (v & 0xF).astype(np.uint8)


def decode_uint4(codes):
    return np.asarray(codes).astype(np.int64) & 0xF


# ---------------------------------------------------------------- E2M1 (FP4)


def decode_e2m1(codes):
    """OCP MX FP4 E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.

    Exponent field 0 is subnormal: value = 0.5 * mantissa. Otherwise
    value = 2**(e-1) * (1 + mantissa/2).
    """
    c = np.asarray(codes).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, (e - 1).astype(np.int32)))
    return sign * mag


_E2M1_POS = decode_e2m1(np.arange(8))  # 0, .5, 1, 1.5, 2, 3, 4, 6 (codes 0..7)


def _nearest_even(mag, table):
    """Index into the increasing ``table`` of the value nearest ``mag`` (>= 0);
    on an exact tie the even index (even code = mantissa LSB 0) wins.
    ``mag`` must lie within [table[0], table[-1]]."""
    mag = np.asarray(mag, dtype=np.float64)
    hi = np.searchsorted(table, mag, side="left")
    hi = np.clip(hi, 0, len(table) - 1)
    lo = np.clip(hi - 1, 0, len(table) - 1)
    d_lo = mag - table[lo]
    d_hi = table[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    return np.where(pick_hi, hi, lo)


def encode_e2m1_rne_sat(x):
    """Real -> E2M1 code, round to nearest (ties to even), saturate at +-6.

    The MX specification converts element values by RNE and clamps values
    beyond the largest normal to it.
    """
    x = np.asarray(x, dtype=np.float64)
    assert not np.any(np.isnan(x))
    mag = np.minimum(np.abs(x), 6.0)
    idx = _nearest_even(mag, _E2M1_POS)
    sign = np.signbit(x).astype(np.int64) << 3
    return (idx | sign).astype(np.uint8)


# ---------------------------------------------------------------- E8M0


def decode_e8m0(codes):
    """E8M0 scale: 2**(e - 127); code 255 is NaN (invalid as a scale)."""
    e = np.asarray(codes).astype(np.int64)
    out = np.ldexp(1.0, (e - 127).astype(np.int32))
    return np.where(e == 255, np.nan, out)


# ---------------------------------------------------------------- E4M3 (OFP8)


def decode_e4m3(codes):
    """OCP E4M3 ("fn" variant): bias 7, S.1111.111 = NaN, no infinities."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = np.ldexp(m / 8.0, -6)
    nrm = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32))
    mag = np.where(e == 0, sub, nrm)
    out = sign * mag
    return np.where((e == 15) & (m == 7), np.nan, out)


_E4M3_POS = decode_e4m3(np.arange(0x7F))  # codes 0x00..0x7E, increasing, max 448


def encode_e4m3_rne(x):
    """Real with |x| <= 448 -> E4M3 code by round-to-nearest-even.

    Callers clamp to +-448 first, so no value can round to NaN. The sign of
    zero is kept (-0.0 -> 0x80).
    """
    x = np.asarray(x, dtype=np.float64)
    assert not np.any(np.isnan(x))
    assert np.all(np.abs(x) <= 448.0), "clamp to +-448 before encoding"
    idx = _nearest_even(np.abs(x), _E4M3_POS)
    sign = np.signbit(x).astype(np.int64) << 7
    return (idx | sign).astype(np.uint8)


# ---------------------------------------------------------------- bf16 / fp16


def bf16_bits_to_f64(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x):
    """binary32 -> bf16 bit pattern, round to nearest even (NaN stays NaN)."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    return np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), r)


def f16_bits_to_f64(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f32_to_f16_bits(x):
    """binary32 -> binary16 bit pattern (numpy's cast: IEEE RNE)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)
