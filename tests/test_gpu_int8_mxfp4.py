"""W8A8, W4A8-INT8 and W4A8-MXFP4 parity against the oracle, plus the
activation quantizers (bit-exact) and the standard-format producer.

Integer accumulators (otype I32) must match the exact integer product bit for
bit. Scaled outputs: relative Frobenius error <= 1e-3 with fp32 output (the
scaled epilogue before any output rounding) and <= 2e-3 with bf16 output.
"""

import numpy as np
import pytest
import torch

import quantized_dequant_gemm_amd as q
import synth
from oracle import codecs, metrics, quant, ref
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _act_int8(m, k, salt=0):
    a = synth.activations_bf16_bits(m, k, workload_id=2, salt=salt)
    qa, sa = quant.quantize_act_int8(a)
    return a, qa, sa


def _run_int(layer, pk, qa, sa, m, tuning=None):
    return H.gemm(layer, pk, H.dev(qa), m, a_scales=H.dev(sa), tuning=tuning)[0]


# ------------------------------------------------------------ activations


@pytest.mark.parametrize("m,k", [(16, 4096), (256, 4096), (37, 7168), (4096, 4096)])
def test_act_quant_int8_bit_exact(qdg, m, k):
    a = synth.activations_bf16_bits(m, k, workload_id=2, salt=m)
    a[min(3, m - 1)] = 0  # an all-zero row
    qa, sa = quant.quantize_act_int8(a)
    layer = q.layer_w8a8(16, k)
    qa_d = torch.empty((m, k), dtype=torch.int8, device="cuda")
    sa_d = torch.empty(m, dtype=torch.float32, device="cuda")
    q.qdg_quantize_act(layer, H.bf16_dev(a).data_ptr(), m, qa_d.data_ptr(), sa_d.data_ptr(), q.current_stream())
    torch.cuda.synchronize()
    assert np.array_equal(qa_d.cpu().numpy(), qa)
    assert np.array_equal(sa_d.cpu().numpy().view(np.uint32), sa.view(np.uint32))


@pytest.mark.parametrize("m,k", [(16, 7168), (512, 2048), (3, 128), (4096, 7168)])
def test_act_quant_fp8_bit_exact(qdg, m, k):
    a = synth.activations_bf16_bits(m, k, workload_id=3, salt=m)
    a[0, :128] = 0  # an all-zero group
    codes, sa = quant.quantize_act_fp8(a)
    layer = q.layer_mxfp4(16, k)
    qa_d = torch.empty((m, k), dtype=torch.uint8, device="cuda")
    sa_d = torch.empty((m, k // 128), dtype=torch.float32, device="cuda")
    q.qdg_quantize_act(layer, H.bf16_dev(a).data_ptr(), m, qa_d.data_ptr(), sa_d.data_ptr(), q.current_stream())
    torch.cuda.synchronize()
    assert np.array_equal(qa_d.cpu().numpy(), codes)
    assert np.array_equal(sa_d.cpu().numpy().view(np.uint32), sa.view(np.uint32))


def test_act_quant_fp8_every_bf16_magnitude(qdg):
    # Every bf16 value of magnitude <= 448, both signs (subnormal and normal
    # E4M3 codes, every tie between two codes, values that round to a signed
    # zero): each 128-group also holds +-448, so its amax is 448, the inverse
    # scale is exactly 1 and the codes are the E4M3 encoding of the inputs
    # themselves, bit for bit as the oracle's encoder gives them.
    pos = np.arange(0, 0x43E1, dtype=np.uint16)
    vals = np.concatenate([pos, pos | np.uint16(0x8000)])
    per = 127
    ngroups = -(-vals.size // per)
    ngroups = -(-ngroups // 8) * 8  # whole rows of 8 groups
    grid = np.zeros((ngroups, 128), dtype=np.uint16)
    grid[:, 0] = np.where(np.arange(ngroups) % 2 == 0, 0x43E0, 0xC3E0)  # +-448
    flat = np.zeros(ngroups * per, dtype=np.uint16)
    flat[: vals.size] = vals
    grid[:, 1:] = flat.reshape(ngroups, per)
    a = grid.reshape(ngroups // 8, 1024)
    m, k = a.shape
    codes, sa = quant.quantize_act_fp8(a)
    assert np.all(sa.view(np.uint32) == np.float32(1.0).view(np.uint32))
    layer = q.layer_mxfp4(16, k)
    qa_d = torch.empty((m, k), dtype=torch.uint8, device="cuda")
    sa_d = torch.empty((m, k // 128), dtype=torch.float32, device="cuda")
    q.qdg_quantize_act(layer, H.bf16_dev(a).data_ptr(), m, qa_d.data_ptr(), sa_d.data_ptr(), q.current_stream())
    torch.cuda.synchronize()
    got = qa_d.cpu().numpy()
    bad = np.argwhere(got != codes)
    assert bad.size == 0, [(hex(a[r, c]), hex(got[r, c]), hex(codes[r, c])) for r, c in bad[:8]]
    assert np.array_equal(sa_d.cpu().numpy().view(np.uint32), sa.view(np.uint32))


# ------------------------------------------------------------ W8A8


@pytest.mark.parametrize("m,n,k", [(16, 4096, 4096), (256, 4096, 4096), (16, 14336, 4096), (5, 200, 384)])
def test_w8a8(qdg, m, n, k):
    w = synth.weights_f32(n, k, workload_id=2, salt=1)
    qw, sw = quant.quantize_int8_per_channel(w)
    a, qa, sa = _act_int8(m, k, salt=m)
    y64, p = ref.gemm_w8a8(qa, sa, qw, sw)
    for otype in (q.QDG_O_I32, q.QDG_O_F32, q.QDG_O_BF16):
        layer = q.layer_w8a8(n, k, otype=otype)
        pk = H.Packed(layer, H.dev(qw.astype(np.int8)), H.dev(sw))
        y = _run_int(layer, pk, qa, sa, m)
        if otype == q.QDG_O_I32:
            assert np.array_equal(y.cpu().numpy().astype(np.int64), p)
        else:
            err = metrics.rel_frob(H.to_f64(y), y64)
            assert err <= (1e-3 if otype == q.QDG_O_F32 else 2e-3), err


# ------------------------------------------------------------ W4A8-INT8


@pytest.mark.parametrize("m,n,k", [(16, 4096, 4096), (256, 4096, 4096), (16, 14336, 4096), (7, 144, 640)])
def test_w4a8_int8(qdg, m, n, k):
    w = synth.weights_f32(n, k, workload_id=2, salt=2)
    qv, s16 = quant.quantize_int4_sym(w)
    a, qa, sa = _act_int8(m, k, salt=m + 1)
    y64, p = ref.gemm_w4a8(qa, sa, qv, s16)
    qw_d, sc_d, _ = H.std_w4(qv, s16)
    for otype in (q.QDG_O_I32, q.QDG_O_F32, q.QDG_O_BF16):
        layer = q.layer_w4a8(n, k, otype=otype)
        pk = H.Packed(layer, qw_d, sc_d)
        y = _run_int(layer, pk, qa, sa, m)
        if otype == q.QDG_O_I32:
            assert np.array_equal(y.cpu().numpy().astype(np.int64), p)
        else:
            err = metrics.rel_frob(H.to_f64(y), y64)
            assert err <= (1e-3 if otype == q.QDG_O_F32 else 2e-3), err


# ------------------------------------------------------------ MXFP4


def _mxfp4_case(m, n, k, salt=0):
    w = synth.weights_f32(n, k, workload_id=3, salt=salt)
    codes, e = quant.quantize_mxfp4(w)
    a = synth.activations_bf16_bits(m, k, workload_id=3, salt=salt + 1)
    ac, sa = quant.quantize_act_fp8(a)
    return codes, e, ac, sa, ref.gemm_mxfp4(ac, sa, codes, e)


@pytest.mark.parametrize("m,n,k", [(16, 2048, 7168), (16, 7168, 2048), (512, 2048, 7168), (512, 7168, 2048),
                                   (9, 80, 256)])
def test_w4a8_mxfp4(qdg, m, n, k):
    codes, e, ac, sa, y64 = _mxfp4_case(m, n, k, salt=m)
    for otype in (q.QDG_O_F32, q.QDG_O_BF16):
        layer = q.layer_mxfp4(n, k, otype=otype)
        pk = H.Packed(layer, H.dev(codecs.pack_nibbles(codes)), H.dev(e))
        y = H.gemm(layer, pk, H.dev(ac), m, a_scales=H.dev(sa))[0]
        err = metrics.rel_frob(H.to_f64(y), y64)
        print(f"MXFP4 M={m} N={n} K={k} otype={otype}: rel_frob={err:.3e}")
        assert err <= (1e-3 if otype == q.QDG_O_F32 else 2e-3), err


def test_mxfp4_one_hot_layout(qdg):
    # fp8 activation 1.0 (code 0x38) on one k with unit scale: Y[:, n] is the
    # dequantized weight -> pins the E2M1 nibble order and the block-scale lanes
    k, n = 256, 32
    w = synth.weights_f32(n, k, workload_id=3, salt=9)
    codes, e = quant.quantize_mxfp4(w)
    ac = np.where(np.eye(k, dtype=bool), 0x38, 0).astype(np.uint8)
    sa = np.ones((k, k // 128), np.float32)
    layer = q.layer_mxfp4(n, k, otype=q.QDG_O_F32)
    pk = H.Packed(layer, H.dev(codecs.pack_nibbles(codes)), H.dev(e))
    y = H.gemm(layer, pk, H.dev(ac), k, a_scales=H.dev(sa))[0]
    assert np.array_equal(H.to_f64(y), ref.dequant_mxfp4(codes, e).T)


# ------------------------------------------------------------ quantizer


@pytest.mark.parametrize("kind", ["int4", "uint4", "int8", "mxfp4"])
def test_quantize_weights_bit_exact(qdg, kind):
    n, k = 96, 1024
    w = synth.weights_f32(n, k, workload_id=1, salt=21)
    w[3, :128] = 0.0  # an all-zero group / block
    wd = H.dev(w)
    if kind in ("int4", "uint4"):
        layer = q.layer_w4a16(n, k, asym=kind == "uint4")
        qw = torch.empty((n, k // 2), dtype=torch.uint8, device="cuda")
        sc = torch.empty((n, k // 128), dtype=torch.int16, device="cuda")
        z = torch.empty((n, k // 128), dtype=torch.uint8, device="cuda")
        q.qdg_quantize_weights(layer, wd.data_ptr(), qw.data_ptr(), sc.data_ptr(), z.data_ptr(), q.current_stream())
        torch.cuda.synchronize()
        if kind == "int4":
            qv, s = quant.quantize_int4_sym(w)
            assert np.array_equal(qw.cpu().numpy(), codecs.pack_nibbles(codecs.encode_int4(qv)))
        else:
            qv, s, zz = quant.quantize_uint4_asym(w)
            assert np.array_equal(qw.cpu().numpy(), codecs.pack_nibbles(qv))
            assert np.array_equal(z.cpu().numpy(), zz)
        assert np.array_equal(sc.cpu().numpy().view(np.uint16), s)
    elif kind == "int8":
        layer = q.layer_w8a8(n, k)
        qw = torch.empty((n, k), dtype=torch.int8, device="cuda")
        sc = torch.empty(n, dtype=torch.float32, device="cuda")
        q.qdg_quantize_weights(layer, wd.data_ptr(), qw.data_ptr(), sc.data_ptr(), None, q.current_stream())
        torch.cuda.synchronize()
        qv, s = quant.quantize_int8_per_channel(w)
        assert np.array_equal(qw.cpu().numpy().astype(np.int64), qv)
        assert np.array_equal(sc.cpu().numpy().view(np.uint32), s.view(np.uint32))
    else:
        layer = q.layer_mxfp4(n, k)
        qw = torch.empty((n, k // 2), dtype=torch.uint8, device="cuda")
        sc = torch.empty((n, k // 32), dtype=torch.uint8, device="cuda")
        q.qdg_quantize_weights(layer, wd.data_ptr(), qw.data_ptr(), sc.data_ptr(), None, q.current_stream())
        torch.cuda.synchronize()
        c, e = quant.quantize_mxfp4(w)
        assert np.array_equal(qw.cpu().numpy(), codecs.pack_nibbles(c))
        assert np.array_equal(sc.cpu().numpy(), e)


# ------------------------------------------------------------ LDS-tiled family (M > 64)


def _int_layer_data(kind, n, k, salt):
    w = synth.weights_f32(n, k, workload_id=2, salt=salt)
    if kind == "w8a8":
        qw, sw = quant.quantize_int8_per_channel(w)
        return dict(qw=qw, sw=sw, std=(H.dev(qw.astype(np.int8)), H.dev(sw)))
    qv, s16 = quant.quantize_int4_sym(w)
    qw_d, sc_d, _ = H.std_w4(qv, s16)
    return dict(qv=qv, s16=s16, std=(qw_d, sc_d))


def _int_ref(kind, d, qa, sa):
    if kind == "w8a8":
        return ref.gemm_w8a8(qa, sa, d["qw"], d["sw"])
    return ref.gemm_w4a8(qa, sa, d["qv"], d["s16"])


def _int_layer(kind, n, k, otype):
    return q.layer_w8a8(n, k, otype=otype) if kind == "w8a8" else q.layer_w4a8(n, k, otype=otype)


def _family(layer, m, tuning=None):
    plan = q.qdg_plan_create(layer, q.dense(), tuning)
    return q.qdg_plan_describe(plan, m).split("family=")[1].split()[0]


@pytest.mark.parametrize("kind", ["w8a8", "w4a8"])
@pytest.mark.parametrize("m,n,k", [(300, 200, 640), (129, 1040, 1024)])
def test_int8_tiled_ragged(qdg, kind, m, n, k):
    # ragged M (partial 128-row tiles), ragged N (a partial 256-column tile)
    # and a split K range through the 8-bit tiled family (pinned by the
    # tuning: at so few tiles the heuristic picks the streaming family)
    d = _int_layer_data(kind, n, k, salt=m)
    a, qa, sa = _act_int8(m, k, salt=m + 7)
    y64, p = _int_ref(kind, d, qa, sa)
    t = q.TuningConfig(block_m=128)
    for otype in (q.QDG_O_I32, q.QDG_O_F32, q.QDG_O_BF16):
        layer = _int_layer(kind, n, k, otype)
        assert _family(layer, m, t) == "qtile"
        pk = H.Packed(layer, *d["std"])
        y = _run_int(layer, pk, qa, sa, m, tuning=t)
        if otype == q.QDG_O_I32:
            assert np.array_equal(y.cpu().numpy().astype(np.int64), p)
        else:
            err = metrics.rel_frob(H.to_f64(y), y64)
            assert err <= (1e-3 if otype == q.QDG_O_F32 else 2e-3), err


@pytest.mark.parametrize("kind", ["w8a8", "w4a8"])
@pytest.mark.parametrize("n", [4096, 14336])
def test_int8_full_size_sampled_rows(qdg, kind, n):
    # M = 4096, K = 4096 as the benchmark runs it; the oracle checks 40
    # sampled rows (every column); raw int32 must match exactly
    m, k = 4096, 4096
    d = _int_layer_data(kind, n, k, salt=n)
    a, qa, sa = _act_int8(m, k, salt=5)
    rows = np.unique(np.concatenate([[0, m - 1], np.random.default_rng(n).integers(0, m, 38)]))
    y64, p = _int_ref(kind, d, qa[rows], sa[rows])
    rows_d = torch.from_numpy(rows).cuda()
    for otype in (q.QDG_O_I32, q.QDG_O_BF16):
        layer = _int_layer(kind, n, k, otype)
        pk = H.Packed(layer, *d["std"])
        y = _run_int(layer, pk, qa, sa, m)
        ys = y[rows_d]
        if otype == q.QDG_O_I32:
            assert np.array_equal(ys.cpu().numpy().astype(np.int64), p)
        else:
            err = metrics.rel_frob(H.to_f64(ys), y64)
            print(f"{kind} M={m} K={k} N={n} sampled rows: rel_frob={err:.3e}")
            assert err <= 2e-3, err
            H.assert_elementwise(ys, y64)
            assert not torch.isnan(y.float()).any()


@pytest.mark.parametrize("kind", ["w8a8", "w4a8", "mxfp4"])
def test_tiled_8bit_split_k_deterministic(qdg, kind):
    m, n, k = 256, 512, 2048
    if kind == "mxfp4":
        codes, e, ac, sa, y64 = _mxfp4_case(m, n, k, salt=31)
        std = (H.dev(codecs.pack_nibbles(codes)), H.dev(e))
        a_d, sa_d = H.dev(ac), H.dev(sa)
        mk = lambda: q.layer_mxfp4(n, k, otype=q.QDG_O_F32)  # noqa: E731
    else:
        d = _int_layer_data(kind, n, k, salt=31)
        a, qa, sa = _act_int8(m, k, salt=32)
        y64, _ = _int_ref(kind, d, qa, sa)
        std = d["std"]
        a_d, sa_d = H.dev(qa), H.dev(sa)
        mk = lambda: _int_layer(kind, n, k, q.QDG_O_F32)  # noqa: E731
    outs = {}
    for split in (1, 3, 8):
        layer = mk()
        t = q.TuningConfig(block_m=128, split_k=split)
        assert _family(layer, m, t) == "qtile"
        pk = H.Packed(layer, *std)
        y1 = H.gemm(layer, pk, a_d, m, a_scales=sa_d, tuning=t)[0]
        y2 = H.gemm(layer, pk, a_d, m, a_scales=sa_d, tuning=t)[0]
        assert torch.equal(y1, y2), f"split {split} not deterministic"
        assert metrics.rel_frob(H.to_f64(y1), y64) <= 1e-3
        outs[split] = H.to_f64(y1)
    assert np.allclose(outs[1], outs[8], rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("k,n", [(7168, 2048), (2048, 7168)])
def test_mxfp4_full_size_sampled_rows(qdg, k, n):
    m = 4096
    codes, e, ac, sa, _ = _mxfp4_case(16, n, k, salt=41)  # weights only; A below
    a = synth.activations_bf16_bits(m, k, workload_id=3, salt=42)
    ac, sa = quant.quantize_act_fp8(a)
    rows = np.unique(np.concatenate([[0, m - 1], np.random.default_rng(k).integers(0, m, 38)]))
    y64 = ref.gemm_mxfp4(ac[rows], sa[rows], codes, e)
    layer = q.layer_mxfp4(n, k)
    assert _family(layer, m) == "qtile"
    pk = H.Packed(layer, H.dev(codecs.pack_nibbles(codes)), H.dev(e))
    y = H.gemm(layer, pk, H.dev(ac), m, a_scales=H.dev(sa))[0]
    ys = y[torch.from_numpy(rows).cuda()]
    err = metrics.rel_frob(H.to_f64(ys), y64)
    print(f"MXFP4 M={m} K={k} N={n} sampled rows: rel_frob={err:.3e}")
    assert err <= 2e-3, err
    H.assert_elementwise(ys, y64)
    assert not torch.isnan(y.float()).any()


# ------------------------------------------------------------ weight streaming (M <= 16)


def _any_case(kind, m, n, k, salt):
    """(layer maker, std tensors, A codes, A scales, Y64, raw P or None)."""
    if kind == "mxfp4":
        codes, e, ac, sa, y64 = _mxfp4_case(m, n, k, salt=salt)
        return (lambda o: q.layer_mxfp4(n, k, otype=o)), (H.dev(codecs.pack_nibbles(codes)), H.dev(e)), ac, sa, y64, None
    d = _int_layer_data(kind, n, k, salt=salt)
    a, qa, sa = _act_int8(m, k, salt=salt + 1)
    y64, p = _int_ref(kind, d, qa, sa)
    return (lambda o: _int_layer(kind, n, k, o)), d["std"], qa, sa, y64, p


@pytest.mark.parametrize("kind", ["w8a8", "w4a8", "mxfp4"])
@pytest.mark.parametrize("m,n,k,pin", [(1, 4096, 4096, False), (3, 272, 1152, False), (3, 272, 1152, True),
                                       (16, 1040, 8320, False)])
def test_8bit_weight_streaming(qdg, kind, m, n, k, pin):
    # M <= 16 through the weight-streaming family: one row, a ragged tile
    # count with a short K (9 groups: the streaming family without a tuning,
    # weight streaming when a tuning pins it), and K = 8320 (65 groups: more
    # than one workgroup holds, so K is split at least in two)
    mk, std, ac, sa, y64, p = _any_case(kind, m, n, k, salt=50 + m)
    otypes = (q.QDG_O_F32, q.QDG_O_BF16) if kind == "mxfp4" else (q.QDG_O_I32, q.QDG_O_F32, q.QDG_O_BF16)
    t = q.TuningConfig(waves=8) if pin else None
    for otype in otypes:
        layer = mk(otype)
        fam = _family(layer, m, t)
        raw = otype == q.QDG_O_I32
        ws = (pin or k // 128 >= 32) and not (raw and k > 8192)
        assert fam == ("wstream" if ws else "stream"), fam
        pk = H.Packed(layer, *std)
        y = H.gemm(layer, pk, H.dev(ac), m, a_scales=H.dev(sa), tuning=t)[0]
        if raw:
            assert np.array_equal(y.cpu().numpy().astype(np.int64), p)
        else:
            err = metrics.rel_frob(H.to_f64(y), y64)
            assert err <= (1e-3 if otype == q.QDG_O_F32 else 2e-3), (otype, err)


@pytest.mark.parametrize("kind", ["w8a8", "w4a8", "mxfp4"])
def test_8bit_weight_streaming_split_k(qdg, kind):
    m, n, k = 16, 512, 4096
    mk, std, ac, sa, y64, _ = _any_case(kind, m, n, k, salt=61)
    outs = {}
    for split in (1, 3, 32):
        layer = mk(q.QDG_O_F32)
        t = q.TuningConfig(split_k=split)
        assert _family(layer, m, t) == "wstream"
        pk = H.Packed(layer, *std)
        y1 = H.gemm(layer, pk, H.dev(ac), m, a_scales=H.dev(sa), tuning=t)[0]
        y2 = H.gemm(layer, pk, H.dev(ac), m, a_scales=H.dev(sa), tuning=t)[0]
        assert torch.equal(y1, y2), f"split {split} not deterministic"
        assert metrics.rel_frob(H.to_f64(y1), y64) <= 1e-3
        outs[split] = H.to_f64(y1)
    assert np.allclose(outs[1], outs[32], rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("kind", ["w8a8", "w4a8", "mxfp4"])
@pytest.mark.parametrize("m,n,k", [(64, 4096, 4096), (100, 528, 2048)])
def test_8bit_tiled_partial_row_block(qdg, kind, m, n, k):
    # 64 <= M < 128: the tiled family with one partly filled 128-row block
    # and K split into one pass of workgroups; integer results stay exact
    # (pinned to 128-row blocks: for narrow int8 x int8 layers the heuristic
    # keeps the streaming family up to 128 rows)
    mk, std, ac, sa, y64, p = _any_case(kind, m, n, k, salt=70 + m)
    otypes = (q.QDG_O_F32, q.QDG_O_BF16) if kind == "mxfp4" else (q.QDG_O_I32, q.QDG_O_F32, q.QDG_O_BF16)
    t = q.TuningConfig(block_m=128)
    for otype in otypes:
        layer = mk(otype)
        assert _family(layer, m, t) == "qtile"
        pk = H.Packed(layer, *std)
        y = H.gemm(layer, pk, H.dev(ac), m, a_scales=H.dev(sa), tuning=t)[0]
        if otype == q.QDG_O_I32:
            assert np.array_equal(y.cpu().numpy().astype(np.int64), p)
        else:
            err = metrics.rel_frob(H.to_f64(y), y64)
            assert err <= (1e-3 if otype == q.QDG_O_F32 else 2e-3), (otype, err)
