"""W2A16 (2-bit asymmetric weights, bf16 activations) on the GPU against the
fp64 oracle, through the streaming family (M <= 32, MoE blocks of 16 to 64
rows) and the LDS-tiled bf16 family (M >= 33, 128-row MoE blocks): every
integer q - z is exact in the bf16 MFMA and the group scale is applied in
fp32, so fp32 output stays within 5e-5 relative Frobenius of the fp64
reference and bf16 output within 2e-3; one-hot rows reproduce every
dequantized weight exactly; the device producer of the standard format
matches the oracle's quantizer bit for bit."""

import numpy as np
import pytest
import torch

import quantized_dequant_gemm_amd as q
import synth
from oracle import codecs, metrics, quant, ref
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _data(n, k, salt):
    w = synth.weights_f32(n, k, workload_id=1, salt=salt)
    qv, s, z = quant.quantize_uint2_asym(w)
    return qv, s, z, ref.dequant_uint2_asym(qv, s, z)


def _packed(n, k, qv, s, z, otype, num_experts=1):
    layer = q.layer_w2a16(n, k, otype=otype, num_experts=num_experts)
    pk = H.Packed(layer, H.dev(codecs.pack_crumbs(qv)), H.dev(np.asarray(s, np.uint16).view(np.int16)), H.dev(z))
    return layer, pk


@pytest.mark.parametrize("m,n,k", [(1, 96, 256), (16, 4096, 4096), (16, 1024, 14336), (37, 200, 640),
                                   (64, 512, 1024), (150, 272, 512), (300, 1040, 2048)])
def test_w2a16_parity(qdg, m, n, k):
    qv, s, z, w64 = _data(n, k, salt=m)
    a = synth.activations_bf16_bits(m, k, workload_id=1, salt=m + 1)
    y64 = ref.gemm_w4a16(a, w64)
    for otype, tol in ((q.QDG_O_F32, 5e-5), (q.QDG_O_BF16, 2e-3)):
        layer, pk = _packed(n, k, qv, s, z, otype)
        y, plan = H.gemm(layer, pk, H.bf16_dev(a), m)
        # the streaming family up to 32 rows, the LDS-tiled bf16 family above
        assert ("family=stream " if m <= 32 else "family=tile ") in q.qdg_plan_describe(plan, m)
        err = metrics.rel_frob(H.to_f64(y), y64)
        print(f"W2A16 M={m} N={n} K={k} otype={otype}: rel_frob={err:.3e}")
        assert err <= tol, err


@pytest.mark.parametrize("m", [16, 64, 128])
def test_w2a16_one_hot_every_code_and_zero(qdg, m):
    # codes and zero points over their whole range, power-of-two scales: one
    # identity row per k returns (q - z) * s exactly (fp32 output)
    k, n = 256, 80
    r = np.random.default_rng(m)
    qv = r.integers(0, 4, (n, k))
    qv[:, :4] = [0, 1, 2, 3]
    z = r.integers(0, 4, (n, k // 128)).astype(np.uint8)
    z[:4, 0] = [0, 1, 2, 3]
    s = codecs.f32_to_f16_bits(np.ldexp(1.0, r.integers(-12, -3, (n, k // 128))).astype(np.float32))
    w64 = ref.dequant_uint2_asym(qv, s, z)
    layer, pk = _packed(n, k, qv, s, z, q.QDG_O_F32)
    for base in range(0, k, m):
        eye = np.zeros((m, k), np.float32)
        eye[np.arange(m), np.arange(base, base + m) % k] = 1.0
        y = H.gemm(layer, pk, H.bf16_dev(codecs.f32_to_bf16_bits(eye)), m)[0]
        cnt = min(m, k - base)
        assert np.array_equal(H.to_f64(y)[:cnt], w64[:, base:base + cnt].T)


def test_w2a16_device_producer_bit_exact(qdg):
    n, k = 272, 1024
    w = synth.weights_f32(n, k, workload_id=1, salt=31)
    w[5, :128] = 0.0  # an all-zero group: scale 1, zero point 0
    qv, s, z = quant.quantize_uint2_asym(w)
    layer = q.layer_w2a16(n, k)
    qw = torch.empty((n, k // 4), dtype=torch.uint8, device="cuda")
    sc = torch.empty((n, k // 128), dtype=torch.int16, device="cuda")
    zz = torch.empty((n, k // 128), dtype=torch.uint8, device="cuda")
    q.qdg_quantize_weights(layer, H.dev(w).data_ptr(), qw.data_ptr(), sc.data_ptr(), zz.data_ptr(),
                           q.current_stream())
    torch.cuda.synchronize()
    assert np.array_equal(qw.cpu().numpy(), codecs.pack_crumbs(qv))
    assert np.array_equal(sc.cpu().numpy().view(np.uint16), s)
    assert np.array_equal(zz.cpu().numpy(), z)


def test_w2a16_zero_point_flag(qdg):
    n, k = 32, 256
    qv, s, z, _ = _data(n, k, salt=3)
    layer = q.layer_w2a16(n, k)
    z2 = z.copy()
    z2[9, 1] = 4
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    nbytes = q.qdg_preprocess_query(layer)
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    qw, sc = H.dev(codecs.pack_crumbs(qv)), H.dev(np.asarray(s, np.uint16).view(np.int16))
    q.qdg_preprocess(layer, q.StdWeights(qw.data_ptr(), sc.data_ptr(), H.dev(z).data_ptr()), buf.data_ptr(), nbytes,
                     q.current_stream(), status=st.data_ptr())
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    q.qdg_preprocess(layer, q.StdWeights(qw.data_ptr(), sc.data_ptr(), H.dev(z2).data_ptr()), buf.data_ptr(),
                     nbytes, q.current_stream(), status=st.data_ptr())
    torch.cuda.synchronize()
    assert int(st.item()) == q.QDG_FLAG_BAD_ZERO_POINT


@pytest.mark.parametrize("bm,t,hid,n", [(16, 70, 512, 192), (32, 70, 512, 192), (64, 70, 512, 192),
                                        (128, 70, 512, 192), (128, 400, 1024, 384)])
def test_w2a16_moe(qdg, bm, t, hid, n):
    E, top_k = 4, 2
    ids, _ = ref.route_topk(synth.router_logits(t, E, salt=bm + 40), top_k)
    data = [_data(n, hid, salt=200 + e) for e in range(E)]
    layer = q.layer_w2a16(n, hid, otype=q.QDG_O_F32, num_experts=E)
    pk = H.Packed(layer, H.dev(np.stack([codecs.pack_crumbs(d[0]) for d in data])),
                  H.dev(np.stack([np.asarray(d[1], np.uint16).view(np.int16) for d in data])),
                  H.dev(np.stack([d[2] for d in data])))
    for per_pair in (0, 1):
        rows = t * top_k if per_pair else t
        a = synth.activations_bf16_bits(rows, hid, workload_id=1, salt=bm + per_pair)
        cap = q.qdg_moe_align_capacity(t, top_k, E, bm)
        sid = torch.empty(cap, dtype=torch.int32, device="cuda")
        blk = torch.empty(cap // bm, dtype=torch.int32, device="cuda")
        npad = torch.zeros(1, dtype=torch.int32, device="cuda")
        q.qdg_moe_align(H.dev(ids.astype(np.int32)).data_ptr(), t, top_k, E, bm, sid.data_ptr(), blk.data_ptr(),
                        npad.data_ptr(), q.current_stream())
        plan = q.qdg_plan_create(layer, q.moe(top_k))
        assert ("family=tile " if bm == 128 else "family=stream ") in q.qdg_moe_describe(plan, t, bm)
        wsp, nbytes = H.workspace(plan, t)
        y = H.out_tensor(t * top_k, n, q.QDG_O_F32)
        a_d = H.bf16_dev(a)
        q.qdg_moe_gemm(plan, a_d.data_ptr(), None, pk.buf.data_ptr(), sid.data_ptr(), blk.data_ptr(),
                       npad.data_ptr(), t, bm, per_pair, y.data_ptr(), wsp.data_ptr(), nbytes, q.current_stream())
        torch.cuda.synchronize()
        y64 = ref.moe_gemm_rows(a, ids, lambda e: data[e][3], input_is_per_pair=bool(per_pair))
        assert not torch.isnan(y).any()
        err = metrics.rel_frob(H.to_f64(y), y64)
        print(f"W2A16 MoE bm={bm} per_pair={per_pair}: rel_frob={err:.3e}")
        assert err <= 5e-5, err
