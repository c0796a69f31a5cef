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


def _run_int(layer, pk, qa, sa, m):
    return H.gemm(layer, pk, H.dev(qa), m, a_scales=H.dev(sa))[0]


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


@pytest.mark.parametrize("m,n,k", [(16, 2048, 7168), (16, 7168, 2048), (512, 2048, 7168), (9, 80, 256)])
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
