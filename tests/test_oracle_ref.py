"""Pins for oracle.ref: closed forms, exact rational brute force, special cases.

Brute force uses Python ``fractions.Fraction`` so it is exact and shares no
arithmetic with numpy/BLAS. A dropped term, a wrong sign of the zero point, a
transposed operand or a misplaced group index in the oracle fails here.
"""

from fractions import Fraction

import numpy as np

import synth
from oracle import codecs, quant, ref


def _frac_f16(bits):
    return Fraction(float(codecs.f16_bits_to_f64(bits)))


def test_dequant_hand_examples():
    s_half = codecs.f32_to_f16_bits(np.float32([0.5]))
    s_quarter = codecs.f32_to_f16_bits(np.float32([0.25]))
    q = np.full((1, 128), 11)
    z = np.array([[8]], np.uint8)
    assert ref.dequant_uint4_asym(q, s_half.reshape(1, 1), z)[0, 0] == 1.5
    qs = np.full((1, 128), -8)
    assert ref.dequant_int4_sym(qs, s_quarter.reshape(1, 1))[0, 0] == -2.0
    # MXFP4: code 0x5 (3.0) with E8M0 126 (0.5) -> 1.5; code 0xF (-6) with 130 (8) -> -48
    c = np.zeros((1, 32), np.uint8)
    c[0, 0], c[0, 1] = 0x5, 0xF
    assert ref.dequant_mxfp4(c, np.array([[126]], np.uint8))[0, :2].tolist() == [1.5, -3.0]
    assert ref.dequant_mxfp4(c, np.array([[130]], np.uint8))[0, 1] == -48.0


def _tiny_w4a16(m, n, k, asym, seed):
    r = np.random.default_rng(seed)
    a = synth.activations_bf16_bits(m, k, workload_id=0, salt=seed)
    s = codecs.f32_to_f16_bits(r.uniform(1e-3, 1e-2, (n, k // 128)).astype(np.float32))
    if asym:
        q = r.integers(0, 16, (n, k))
        z = r.integers(0, 16, (n, k // 128)).astype(np.uint8)
        w = ref.dequant_uint4_asym(q, s, z)
    else:
        q = r.integers(-8, 8, (n, k))
        z = np.zeros((n, k // 128), np.uint8)
        w = ref.dequant_int4_sym(q, s)
    return a, q, s, z, w


def test_w4a16_brute_force_exact():
    for asym in (False, True):
        m, n, k = 3, 4, 256
        a, q, s, z, w = _tiny_w4a16(m, n, k, asym, seed=5 + asym)
        y = ref.gemm_w4a16(a, w)
        af = [[Fraction(float(v)) for v in row] for row in codecs.bf16_bits_to_f64(a)]
        for i in range(m):
            for j in range(n):
                acc = Fraction(0)
                for kk in range(k):
                    g = kk // 128
                    acc += af[i][kk] * (int(q[j, kk]) - int(z[j, g])) * _frac_f16(s[j, g])
                # float64 BLAS over exact float64 products: tiny relative error only
                assert abs(float(acc) - y[i, j]) <= 1e-12 * max(1.0, abs(float(acc)))


def test_w4a16_one_hot_recovers_weights():
    m, n, k = 256, 8, 256
    a, q, s, z, w = _tiny_w4a16(1, n, k, True, seed=9)
    eye = codecs.f32_to_bf16_bits(np.eye(k, dtype=np.float32))
    y = ref.gemm_w4a16(eye, w)
    assert np.array_equal(y, w.T)


def test_w4a16_special_cases():
    a, q, s, z, w = _tiny_w4a16(4, 8, 384, False, seed=13)
    y = ref.gemm_w4a16(a, w)
    # power-of-two scaling of every scale doubles Y exactly
    s2 = codecs.f32_to_f16_bits(codecs.f16_bits_to_f64(s).astype(np.float32) * 2)
    assert np.array_equal(ref.gemm_w4a16(a, ref.dequant_int4_sym(q, s2)), 2 * y)
    # unit scales reduce to an exact integer matmul
    ones = codecs.f32_to_f16_bits(np.ones_like(s, dtype=np.float32))
    yi = ref.gemm_w4a16(a, ref.dequant_int4_sym(q, ones))
    af = codecs.bf16_bits_to_f64(a)
    exact = [[sum(Fraction(float(af[i, kk])) * int(q[j, kk]) for kk in range(384))
              for j in range(8)] for i in range(4)]
    assert np.allclose(yi, np.array(exact, dtype=np.float64), rtol=1e-13, atol=0)
    # M = 1 is the GEMV of a row
    assert np.allclose(ref.gemm_w4a16(a[1:2], w)[0], y[1], rtol=1e-14)


def test_integer_gemms_exact():
    r = np.random.default_rng(20)
    qa = r.integers(-127, 128, (5, 4096)).astype(np.int8)
    qa[0, :] = 127
    qw = r.integers(-127, 128, (6, 4096)).astype(np.int8)
    qw[0, :] = 127
    sa = r.uniform(0.01, 0.1, 5).astype(np.float32)
    sw = r.uniform(1e-4, 1e-3, 6).astype(np.float32)
    y, p = ref.gemm_w8a8(qa, sa, qw, sw)
    # worst case 4096*127*127 is representable; compare with Python ints
    exact = [[sum(int(qa[i, kk]) * int(qw[j, kk]) for kk in range(4096)) for j in range(6)] for i in range(5)]
    assert p.tolist() == exact
    assert p[0, 0] == 4096 * 127 * 127
    assert np.array_equal(p, ref.int_matmul(qa, qw))
    assert np.allclose(y, p * sa[:, None].astype(np.float64) * sw[None, :], rtol=1e-15)


def test_w4a8_group_scales_brute_force():
    r = np.random.default_rng(21)
    m, n, k = 2, 3, 384
    qa = r.integers(-127, 128, (m, k)).astype(np.int8)
    sa = r.uniform(0.01, 0.1, m).astype(np.float32)
    q = r.integers(-8, 8, (n, k))
    sw = codecs.f32_to_f16_bits(r.uniform(1e-3, 1e-2, (n, k // 128)).astype(np.float32))
    y, p = ref.gemm_w4a8(qa, sa, q, sw)
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            tot = 0
            for g in range(k // 128):
                part = sum(int(qa[i, kk]) * int(q[j, kk]) for kk in range(128 * g, 128 * g + 128))
                acc += _frac_f16(sw[j, g]) * part
                tot += part
            acc *= Fraction(float(sa[i]))
            assert abs(float(acc) - y[i, j]) <= 1e-13 * abs(float(acc)) + 1e-300
            assert p[i, j] == tot


def test_mxfp4_gemm_brute_force():
    r = np.random.default_rng(22)
    m, n, k = 2, 3, 256
    a_codes = r.integers(0, 0x7F, (m, k)).astype(np.uint8) | (r.integers(0, 2, (m, k)) << 7).astype(np.uint8)
    sa = r.uniform(1e-3, 1e-2, (m, k // 128)).astype(np.float32)
    w_codes = r.integers(0, 16, (n, k)).astype(np.uint8)
    e = r.integers(115, 125, (n, k // 32)).astype(np.uint8)
    y = ref.gemm_mxfp4(a_codes, sa, w_codes, e)
    av = codecs.decode_e4m3(a_codes)
    wv = codecs.decode_e2m1(w_codes)
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for kk in range(k):
                acc += (Fraction(float(av[i, kk])) * Fraction(float(sa[i, kk // 128]))
                        * Fraction(float(wv[j, kk])) * Fraction(2) ** (int(e[j, kk // 32]) - 127))
            assert abs(float(acc) - y[i, j]) <= 1e-12 * abs(float(acc)) + 1e-300


def test_w8a16_gemm_brute_force_and_one_hot():
    # exact rationals: bf16 activations times q * s (s fp32), summed exactly
    r = np.random.default_rng(25)
    m, n, k = 2, 3, 64
    a = codecs.f32_to_bf16_bits(r.standard_normal((m, k)).astype(np.float32))
    qw = r.integers(-127, 128, (n, k))
    sw = r.uniform(1e-3, 1e-2, n).astype(np.float32)
    y = ref.gemm_w8a16(a, qw, sw)
    av = codecs.bf16_bits_to_f64(a)
    for i in range(m):
        for j in range(n):
            acc = sum(Fraction(float(av[i, kk])) * int(qw[j, kk]) for kk in range(k)) * Fraction(float(sw[j]))
            assert abs(float(acc) - y[i, j]) <= 1e-12 * abs(float(acc)) + 1e-300
    # one-hot activations return every dequantized weight exactly
    eye = codecs.f32_to_bf16_bits(np.eye(k, dtype=np.float32))
    assert np.array_equal(ref.gemm_w8a16(eye, qw, sw), (qw * sw.astype(np.float64)[:, None]).T)


def test_w4a4_gemm_brute_force():
    # every product e2m1 * e2m1 * 2**(Ea + Eb - 254) is a short dyadic number;
    # the exact rational sum must equal the float64 reference
    r = np.random.default_rng(23)
    m, n, k = 3, 4, 96
    a_codes = r.integers(0, 16, (m, k)).astype(np.uint8)
    w_codes = r.integers(0, 16, (n, k)).astype(np.uint8)
    ea = r.integers(124, 131, (m, k // 32)).astype(np.uint8)
    ew = r.integers(124, 131, (n, k // 32)).astype(np.uint8)
    y = ref.gemm_w4a4(a_codes, ea, w_codes, ew)
    av = codecs.decode_e2m1(a_codes)
    wv = codecs.decode_e2m1(w_codes)
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for kk in range(k):
                acc += (Fraction(float(av[i, kk])) * Fraction(float(wv[j, kk]))
                        * Fraction(2) ** (int(ea[i, kk // 32]) + int(ew[j, kk // 32]) - 254))
            assert float(acc) == y[i, j]


def test_w4a4_special_cases():
    # unit scales (code 127): the product of the decoded E2M1 matrices; a
    # power-of-two activation scale scales the result exactly
    r = np.random.default_rng(24)
    a_codes = r.integers(0, 16, (2, 64)).astype(np.uint8)
    w_codes = r.integers(0, 16, (5, 64)).astype(np.uint8)
    one_a = np.full((2, 2), 127, np.uint8)
    one_w = np.full((5, 2), 127, np.uint8)
    y = ref.gemm_w4a4(a_codes, one_a, w_codes, one_w)
    assert np.array_equal(y, codecs.decode_e2m1(a_codes) @ codecs.decode_e2m1(w_codes).T)
    y3 = ref.gemm_w4a4(a_codes, one_a + 3, w_codes, one_w)
    assert np.array_equal(y3, 8.0 * y)


def test_route_topk_order_and_ties():
    logits = np.array([[0.0, 2.0, 2.0, 1.0], [5.0, -1.0, 5.0, 5.0]])
    ids, p = ref.route_topk(logits, 2)
    assert ids.tolist() == [[1, 2], [0, 2]]
    assert np.all(np.diff(p, axis=1) <= 0)


def test_moe_align_hand_example():
    # pairs: t0 -> (1, 0), t1 -> (1, 2); flat ids 0..3 = (t0j0, t0j1, t1j0, t1j1)
    topk = np.array([[1, 0], [1, 2]])
    sid, blk, npad = ref.moe_align(topk, num_experts=3, block_m=2)
    # expert 0: [1, pad]; expert 1: [0, 2]; expert 2: [3, pad]; sentinel = 4
    assert sid.tolist() == [1, 4, 0, 2, 3, 4]
    assert blk.tolist() == [0, 1, 2]
    assert npad == 6


def test_moe_align_invariants():
    ids, _ = ref.route_topk(synth.router_logits(512, 256), 8)
    for bm in (16, 32, 64):
        sid, blk, npad = ref.moe_align(ids, 256, bm)
        total = ids.size
        real = sid[sid < total]
        assert np.array_equal(np.sort(real), np.arange(total))  # each pair once
        counts = np.bincount(ids.reshape(-1), minlength=256)
        padded = -(-counts // bm) * bm
        assert npad == padded.sum() and npad % bm == 0
        off = np.concatenate([[0], np.cumsum(padded)[:-1]])
        flat = ids.reshape(-1)
        for e in range(256):
            seg = sid[off[e]:off[e] + padded[e]]
            mem = seg[seg < total]
            assert np.all(flat[mem] == e) and np.all(np.diff(mem) > 0)
            assert np.all(seg[len(mem):] == total)
            assert np.all(blk[off[e] // bm:(off[e] + padded[e]) // bm] == e)


def test_moe_gemm_rows_reduces_to_dense():
    t, top_k, n, k = 6, 2, 16, 256
    x = synth.activations_bf16_bits(t, k, workload_id=4, salt=1)
    r = np.random.default_rng(30)
    ws = {e: ref.dequant_int4_sym(r.integers(-8, 8, (n, k)),
                                  codecs.f32_to_f16_bits(r.uniform(1e-3, 1e-2, (n, 2)).astype(np.float32)))
          for e in range(3)}
    ids = np.array([[0, 1], [2, 0], [1, 1], [0, 2], [2, 2], [1, 0]])
    y = ref.moe_gemm_rows(x, ids, lambda e: ws[e], input_is_per_pair=False)
    xf = codecs.bf16_bits_to_f64(x)
    for tt in range(t):
        for j in range(top_k):
            assert np.allclose(y[tt * top_k + j], xf[tt] @ ws[ids[tt, j]].T, rtol=1e-14, atol=0)
    # E = 1 (everything routed to one expert) equals the dense GEMM on repeated rows
    y1 = ref.moe_gemm_rows(x, np.zeros((t, 1), int), lambda e: ws[0], input_is_per_pair=False)
    assert np.array_equal(y1, ref.gemm_w4a16(x, ws[0]))
    # down projection reads one input row per pair
    h = synth.moe_hidden_bf16_bits(t * top_k, k)
    yd = ref.moe_gemm_rows(h, ids, lambda e: ws[e], input_is_per_pair=True)
    hf = codecs.bf16_bits_to_f64(h)
    assert np.allclose(yd[5], hf[5] @ ws[ids[2, 1]].T, rtol=1e-14, atol=0)


def test_moe_rows_brute_force_integer_experts():
    # the format-generic grouped reference against exact per-pair brute force
    # (Python integers): token rows for gate+up, one row per pair for down,
    # with the integer accumulator carried through
    t, top_k, n, k = 5, 3, 4, 32
    r = np.random.default_rng(31)
    qa = r.integers(-127, 128, (t * top_k, k))
    sa = r.uniform(0.5, 2.0, t * top_k)
    qw = {e: r.integers(-127, 128, (n, k)) for e in range(4)}
    sw = {e: r.uniform(0.5, 2.0, n) for e in range(4)}
    ids = np.array([[0, 3, 1], [2, 2, 0], [3, 1, 1], [0, 0, 2], [1, 3, 3]])
    for per_pair in (0, 1):
        y, p = ref.moe_rows(ids, per_pair, lambda e, rows: ref.gemm_w8a8(qa[rows], sa[rows], qw[e], sw[e]))
        for tt in range(t):
            for j in range(top_k):
                i = tt * top_k + j
                row = i if per_pair else tt
                e = int(ids[tt, j])
                for c in range(n):
                    acc = sum(int(qa[row, kk]) * int(qw[e][c, kk]) for kk in range(k))
                    assert p[i, c] == acc
                    assert y[i, c] == acc * sa[row] * sw[e][c]
    # a format without an integer accumulator returns P = None
    y2, p2 = ref.moe_rows(ids, 0, lambda e, rows: np.ones((len(rows), 2)) * e)
    assert p2 is None and np.array_equal(y2[:, 0], ids.reshape(-1).astype(float))


def test_silu_mul_closed_forms():
    # silu(0) = 0, silu(1) = 1 / (1 + e^-1), silu(-x) = silu(x) - x, saturation
    # to x and to 0, and the gate / up column split
    g = np.array([[0.0, 1.0, -1.0, 60.0, -60.0, 2.5]])
    u = np.array([[3.0, 2.0, 2.0, 0.5, 7.0, -1.0]])
    h = ref.silu_mul(np.concatenate([g, u], axis=1))
    s1 = 1.0 / (1.0 + np.exp(-1.0))
    assert h.shape == (1, 6)
    assert h[0, 0] == 0.0
    assert abs(h[0, 1] - 2.0 * s1) <= 1e-15
    assert abs(h[0, 2] - 2.0 * (s1 - 1.0)) <= 1e-15  # silu(-1) = silu(1) - 1
    assert abs(h[0, 3] - 30.0) <= 1e-12 and abs(h[0, 4]) <= 1e-20
    assert abs(h[0, 5] - (-2.5 / (1.0 + np.exp(-2.5)))) <= 1e-15
    # x * sigmoid(x) against the plain formula on random values
    r = np.random.default_rng(33)
    y = r.normal(size=(5, 8))
    hh = ref.silu_mul(y)
    assert np.allclose(hh, y[:, :4] / (1.0 + np.exp(-y[:, :4])) * y[:, 4:], rtol=1e-14, atol=0)


def test_moe_combine_brute_force():
    t, top_k, n = 3, 4, 5
    r = np.random.default_rng(34)
    y = r.integers(-9, 10, (t * top_k, n)).astype(np.float64)
    w = r.integers(1, 5, t * top_k).astype(np.float64)
    out = ref.moe_combine(y, w, top_k)
    for tt in range(t):
        for c in range(n):
            assert out[tt, c] == sum(w[tt * top_k + j] * y[tt * top_k + j, c] for j in range(top_k))


def test_tiny_workload_oracle_shapes():
    # the tiny W4A16 workload end to end through the oracle
    a = synth.activations_bf16_bits(16, 1024, workload_id=0)
    w = synth.weights_f32(512, 1024, workload_id=0)
    q, s, z = quant.quantize_uint4_asym(w)
    y = ref.gemm_w4a16(a, ref.dequant_uint4_asym(q, s, z))
    assert y.shape == (16, 512)
    # 4-bit quantization noise: step ~ range/15 ~ 0.35 sigma, noise ~ step/sqrt(12) ~ 0.1 sigma
    y_fp = codecs.bf16_bits_to_f64(a) @ w.astype(np.float64).T
    assert np.linalg.norm(y - y_fp) / np.linalg.norm(y_fp) < 0.15


def test_mxfp4_int8_gemm_brute_force_and_special_cases():
    # exact rationals: int8 codes times e2m1 * 2**(E-127), times the token scale
    r = np.random.default_rng(26)
    m, n, k = 3, 4, 96
    qa = r.integers(-128, 128, (m, k))
    qa[0, :3] = [-128, 127, 0]
    sa = r.uniform(1e-3, 1e-1, m).astype(np.float32)
    w_codes = r.integers(0, 16, (n, k)).astype(np.uint8)
    e = r.integers(118, 136, (n, k // 32)).astype(np.uint8)
    y = ref.gemm_mxfp4_int8(qa, sa, w_codes, e)
    wv = codecs.decode_e2m1(w_codes)
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for kk in range(k):
                acc += int(qa[i, kk]) * Fraction(float(wv[j, kk])) * Fraction(2) ** (int(e[j, kk // 32]) - 127)
            acc *= Fraction(float(sa[i]))
            assert abs(float(acc) - y[i, j]) <= 1e-15 * abs(float(acc)) + 1e-300
    # unit block scales and token scales: half the exact integer product with
    # the doubled E2M1 values (2 * e2m1 is an integer)
    one = np.full((n, k // 32), 127, np.uint8)
    twice = (2 * wv).astype(np.int64)
    assert np.array_equal(ref.gemm_mxfp4_int8(qa, np.ones(m, np.float32), w_codes, one),
                          ref.int_matmul(qa, twice) / 2.0)
    # a block scale one step up doubles the result exactly; one-hot rows with
    # unit token scale return the dequantized weights
    assert np.array_equal(ref.gemm_mxfp4_int8(qa, sa, w_codes, e + 1), 2.0 * y)
    eye = np.eye(k, dtype=np.int64)
    assert np.array_equal(ref.gemm_mxfp4_int8(eye, np.ones(k, np.float32), w_codes, e),
                          ref.dequant_mxfp4(w_codes, e).T)
    # linear in the activations: negating them negates the result exactly
    assert np.array_equal(ref.gemm_mxfp4_int8(-qa[1:], sa[1:], w_codes, e), -y[1:])


def test_w2a16_dequant_hand_values_and_brute_force():
    # hand values: q = 3, z = 1, s = 0.5 -> 1.0; q = 0, z = 2, s = 0.25 -> -0.5
    s = codecs.f32_to_f16_bits(np.array([[0.5], [0.25]], np.float32))
    q = np.zeros((2, 128), np.int64)
    q[0, 0], q[1, 0] = 3, 0
    z = np.array([[1], [2]], np.uint8)
    w = ref.dequant_uint2_asym(q, s, z)
    assert w[0, 0] == 1.0 and w[1, 0] == -0.5 and w[0, 1] == -0.5 and w[1, 1] == -0.5
    # exact rational brute force of the bf16-activation GEMM on every code and zero point
    r = np.random.default_rng(27)
    m, n, k = 2, 4, 256
    a = codecs.f32_to_bf16_bits(r.standard_normal((m, k)).astype(np.float32))
    qv = r.integers(0, 4, (n, k))
    zz = r.integers(0, 4, (n, k // 128)).astype(np.uint8)
    ss = codecs.f32_to_f16_bits(r.uniform(1e-3, 1e-2, (n, k // 128)).astype(np.float32))
    y = ref.gemm_w4a16(a, ref.dequant_uint2_asym(qv, ss, zz))
    av = codecs.bf16_bits_to_f64(a)
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for kk in range(k):
                acc += (Fraction(float(av[i, kk])) * (int(qv[j, kk]) - int(zz[j, kk // 128]))
                        * _frac_f16(ss[j, kk // 128]))
            assert abs(float(acc) - y[i, j]) <= 1e-12 * abs(float(acc)) + 1e-300
