"""Producers of the standard format and the activation quantizers.

Test infrastructure (see the package docstring).

The pages list the knobs -- integer or floating 4-bit codes, per-group or
per-block scales, symmetric or asymmetric quantization, group size, scale
representation (jetabc, section on what quantization is; kinachrichten,
"Warum quantisierte Kernel wichtig sind") -- but no formula. Readings taken:

* Every decision that turns a real into an integer code is made in IEEE
  binary32 (``np.float32`` arithmetic, correctly rounded division, RNE), so a
  device implementation that does the same binary32 steps reaches the same
  codes bit for bit.
* Symmetric int4: ``s = f16(f32(amax / 7))``, ``q = clamp(rne(f32(w / s)), -8, 7)``.
* Asymmetric uint4: ``s = f16(f32(f32(max - min) / 15))``,
  ``z = clamp(rne(f32(-min / s)), 0, 15)``, ``q = clamp(rne(f32(w / s)) + z, 0, 15)``.
  The range is the group's own min/max (zero is not forced into it).
* Both use the *stored* (fp16-rounded) scale for the codes, so that
  ``deq(quant(w))`` uses exactly the scale a kernel sees. A scale that rounds
  to zero (an all-zero group) is replaced by 1.0.
* int8 per output channel: ``s = f32(amax / 127)`` (fp32 scale),
  ``q = clamp(rne(f32(w / s)), -127, 127)``.
* MXFP4 per OCP MX v1.0: per 32 consecutive K, ``X = floor(log2(amax)) - 2``
  (2 = largest E2M1 exponent), clamped to [-127, 127], stored as ``E = X + 127``;
  elements are ``e2m1_rne_sat(w / 2**X)``. An all-zero block stores ``E = 0``.
* Activations, int8 per token: ``amax`` over the row (exact), ``inv = f32(127 / amax)``,
  ``qa = clamp(rne(f32(x * inv)), -127, 127)``, stored scale ``sa = f32(amax / 127)``.
* Activations, fp8 E4M3 per (token, 128-wide K group): ``inv = f32(448 / amax)``,
  ``qa = e4m3_rne(clamp(f32(x * inv), -448, 448))``, ``sa = f32(amax / 448)``.
* A row or group whose ``amax`` is zero gets scale 1.0 and all-zero codes.
* Activations, MXFP4 (W4A4): the MXFP4 rule above applied to each row's
  blocks of 32 consecutive K (the bf16 values are exact in binary32).
* NVFP4 (named beside INT4 as a 4-bit format with its own number format and
  scaling: kinachrichten, "Warum quantisierte Kernel wichtig sind"; the
  pages give no recipe, so the public NVFP4 definition is taken): E2M1
  elements, one E4M3 scale per 16 consecutive K, one binary32 scale per
  tensor. ``ts = f32(amax_tensor / 2688)`` (2688 = 6 * 448, the largest E2M1
  times the largest E4M3), 1.0 for an all-zero tensor;
  ``sb = e4m3_rne(min(f32(f32(amax_block / 6) / ts), 448))``;
  ``q = e2m1_rne_sat(f32(w / f32(e4m3(sb) * ts)))``, all-zero codes where the
  block scale is zero.
"""

import numpy as np

from . import codecs

F32 = np.float32


def _grouped(w, group):
    n, k = w.shape
    assert k % group == 0, "K must be a multiple of the group size"
    return w.reshape(n, k // group, group)


def _f32_rne(x):
    """RNE of float32 values to integers (numpy rint rounds half to even)."""
    return np.rint(np.asarray(x, dtype=F32))


def quantize_int4_sym(w, group=128):
    """w f32 [N, K] -> (codes int8-valued [N,K] in [-8,7], scales f16 bits [N, K/G])."""
    w = np.asarray(w, dtype=F32)
    wg = _grouped(w, group)
    amax = np.max(np.abs(wg), axis=2)                       # exact
    s32 = (amax / F32(7.0)).astype(F32)                     # f32 division, RNE
    s16 = codecs.f32_to_f16_bits(s32)
    s = codecs.f16_bits_to_f64(s16).astype(F32)
    zero = s == 0
    s = np.where(zero, F32(1.0), s).astype(F32)
    s16 = np.where(zero, codecs.f32_to_f16_bits(np.ones_like(s32)), s16).astype(np.uint16)
    q = _f32_rne((wg / s[:, :, None]).astype(F32))
    q = np.clip(q, -8, 7).astype(np.int64)
    return q.reshape(w.shape), s16


def quantize_uint4_asym(w, group=128):
    """w f32 [N, K] -> (codes [N,K] in [0,15], scales f16 bits [N,K/G], zeros u8 [N,K/G])."""
    w = np.asarray(w, dtype=F32)
    wg = _grouped(w, group)
    mn = np.min(wg, axis=2)
    mx = np.max(wg, axis=2)
    rng = (mx - mn).astype(F32)
    s32 = (rng / F32(15.0)).astype(F32)
    s16 = codecs.f32_to_f16_bits(s32)
    s = codecs.f16_bits_to_f64(s16).astype(F32)
    zero = s == 0
    s = np.where(zero, F32(1.0), s).astype(F32)
    s16 = np.where(zero, codecs.f32_to_f16_bits(np.ones_like(s32)), s16).astype(np.uint16)
    z = np.clip(_f32_rne((-mn / s).astype(F32)), 0, 15).astype(np.int64)
    q = _f32_rne((wg / s[:, :, None]).astype(F32)) + z[:, :, None]
    q = np.clip(q, 0, 15).astype(np.int64)
    return q.reshape(w.shape), s16, z.astype(np.uint8)


def quantize_uint2_asym(w, group=128):
    """w f32 [N, K] -> (codes [N,K] in [0,3], scales f16 bits [N,K/G], zeros u8 [N,K/G]).

    The asymmetric rule of ``quantize_uint4_asym`` with 2-bit codes (the
    pages list WNA16 without fixing N: kinachrichten, "Warum quantisierte
    Kernel wichtig sind"): ``s = f16(f32(max - min) / 3)``,
    ``z = clamp(rne(f32(-min / s)), 0, 3)``, ``q = clamp(rne(f32(w / s)) + z, 0, 3)``,
    with the stored scale; a zero range stores s = 1.
    """
    w = np.asarray(w, dtype=F32)
    wg = _grouped(w, group)
    mn = np.min(wg, axis=2)
    mx = np.max(wg, axis=2)
    s32 = ((mx - mn).astype(F32) / F32(3.0)).astype(F32)
    s16 = codecs.f32_to_f16_bits(s32)
    s = codecs.f16_bits_to_f64(s16).astype(F32)
    zero = s == 0
    s = np.where(zero, F32(1.0), s).astype(F32)
    s16 = np.where(zero, codecs.f32_to_f16_bits(np.ones_like(s32)), s16).astype(np.uint16)
    z = np.clip(_f32_rne((-mn / s).astype(F32)), 0, 3).astype(np.int64)
    q = _f32_rne((wg / s[:, :, None]).astype(F32)) + z[:, :, None]
    q = np.clip(q, 0, 3).astype(np.int64)
    return q.reshape(w.shape), s16, z.astype(np.uint8)


def quantize_int8_per_channel(w):
    """w f32 [N, K] -> (codes int [N,K] in [-127,127], scales f32 [N])."""
    w = np.asarray(w, dtype=F32)
    amax = np.max(np.abs(w), axis=1)
    s = (amax / F32(127.0)).astype(F32)
    s = np.where(s == 0, F32(1.0), s).astype(F32)
    q = np.clip(_f32_rne((w / s[:, None]).astype(F32)), -127, 127).astype(np.int64)
    return q, s


def _floor_log2_f32(a):
    """floor(log2(a)) for positive finite binary32 values, from the bits."""
    a = np.asarray(a, dtype=F32)
    u = a.view(np.uint32).astype(np.int64)
    e = (u >> 23) & 0xFF
    mant = u & 0x7FFFFF
    # subnormal: value = mant * 2**-149 -> floor(log2) = bit_length(mant) - 150
    bl = np.zeros_like(mant)
    m = mant.copy()
    for _ in range(23):
        bl += (m > 0)
        m >>= 1
    return np.where(e == 0, bl - 150, e - 127)


def quantize_mxfp4(w, block=32):
    """w f32 [N, K] -> (E2M1 codes u8 [N,K], E8M0 scale codes u8 [N, K/32])."""
    w = np.asarray(w, dtype=F32)
    wb = _grouped(w, block)
    amax = np.max(np.abs(wb), axis=2)
    pos = amax > 0
    x = np.where(pos, _floor_log2_f32(np.where(pos, amax, F32(1.0))) - 2, -127)
    x = np.clip(x, -127, 127)
    e = (x + 127).astype(np.uint8)
    # w / 2**X is exact for these magnitudes (a power-of-two scaling of a
    # binary32 value whose result stays within binary64 range).
    scaled = wb.astype(np.float64) * np.ldexp(1.0, (-x).astype(np.int32))[:, :, None]
    codes = codecs.encode_e2m1_rne_sat(scaled)
    codes = np.where(pos[:, :, None], codes, 0).astype(np.uint8)
    return codes.reshape(w.shape), e


def quantize_act_mxfp4(a_bf16_bits):
    """bf16 bits [M, K] -> (E2M1 codes u8 [M,K], E8M0 scale codes u8 [M, K/32]).

    MX FP4 activations for the W4A4 path: the same shared-exponent rule and
    element rounding as the weights, one block per 32 consecutive K of a row.
    """
    x = codecs.bf16_bits_to_f64(a_bf16_bits).astype(F32)
    return quantize_mxfp4(x)


def quantize_act_int8(a_bf16_bits):
    """bf16 bits [M, K] -> (qa int8 [M,K], sa f32 [M])."""
    x = codecs.bf16_bits_to_f64(a_bf16_bits).astype(F32)
    amax = np.max(np.abs(x), axis=1).astype(F32)
    nz = amax > 0
    safe = np.where(nz, amax, F32(1.0)).astype(F32)
    inv = (F32(127.0) / safe).astype(F32)
    q = np.clip(_f32_rne((x * inv[:, None]).astype(F32)), -127, 127)
    q = np.where(nz[:, None], q, 0).astype(np.int8)
    sa = np.where(nz, (amax / F32(127.0)).astype(F32), F32(1.0)).astype(F32)
    return q, sa


def quantize_act_fp8(a_bf16_bits, group=128):
    """bf16 bits [M, K] -> (E4M3 codes u8 [M,K], sa f32 [M, K/group])."""
    x = codecs.bf16_bits_to_f64(a_bf16_bits).astype(F32)
    m, k = x.shape
    assert k % group == 0
    xg = x.reshape(m, k // group, group)
    amax = np.max(np.abs(xg), axis=2).astype(F32)
    nz = amax > 0
    safe = np.where(nz, amax, F32(1.0)).astype(F32)
    inv = (F32(448.0) / safe).astype(F32)
    v = (xg * inv[:, :, None]).astype(F32)
    v = np.clip(v, F32(-448.0), F32(448.0))
    codes = codecs.encode_e4m3_rne(v)
    codes = np.where(nz[:, :, None], codes, 0).astype(np.uint8)
    sa = np.where(nz, (amax / F32(448.0)).astype(F32), F32(1.0)).astype(F32)
    return codes.reshape(m, k), sa


def quantize_nvfp4(w, block=16):
    """w f32 [N, K] -> (E2M1 codes u8 [N,K], E4M3 scale codes u8 [N, K/16],
    tensor scale f32)."""
    w = np.asarray(w, dtype=F32)
    amax_t = F32(np.max(np.abs(w))) if w.size else F32(0.0)
    ts = (amax_t / F32(2688.0)).astype(F32) if amax_t > 0 else F32(1.0)
    if ts == 0:  # a tensor amax below 2688 * (smallest subnormal)
        ts = F32(1.0)
    wb = _grouped(w, block)
    amax = np.max(np.abs(wb), axis=2).astype(F32)
    r = ((amax / F32(6.0)).astype(F32) / ts).astype(F32)
    sb = codecs.encode_e4m3_rne(np.minimum(r.astype(np.float64), 448.0))
    den = (codecs.decode_e4m3(sb).astype(F32) * ts).astype(F32)
    nz = den > 0
    scaled = (wb / np.where(nz, den, F32(1.0))[:, :, None]).astype(F32)
    codes = codecs.encode_e2m1_rne_sat(scaled)
    codes = np.where(nz[:, :, None], codes, 0).astype(np.uint8)
    return codes.reshape(w.shape), sb, F32(ts)
