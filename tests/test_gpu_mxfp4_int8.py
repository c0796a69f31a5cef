"""MXFP4 weights x per-token int8 activations (the MXFP4 -> INT8 path) on the
GPU against the fp64 oracle (oracle.ref.gemm_mxfp4_int8), through the
streaming family (M < 64, MoE blocks of 16 and 32 rows) and the 8-bit
LDS-tiled family (M >= 64, MoE blocks of 64 and 128 rows).

The kernel splits every int8 activation exactly into 16 * hi + lo (E4M3
planes) and runs the fp8 x fp4 scaled MFMA on both planes, so every product
is exact and only the fp32 sums round: fp32 output within 1e-3 relative
Frobenius of the fp64 reference, bf16 output within 2e-3, and one-hot rows
(a single nonzero code, unit token scale) reproduce code * weight exactly.
"""

import numpy as np
import pytest
import torch

import quantized_dequant_gemm_amd as q
import synth
from oracle import codecs, metrics, quant, ref
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _weights(n, k, salt):
    w = synth.weights_f32(n, k, workload_id=3, salt=salt)
    return quant.quantize_mxfp4(w)


def _packed(n, k, codes, e, otype, num_experts=1):
    layer = q.layer_mxfp4_int8(n, k, otype=otype, num_experts=num_experts)
    return layer, H.Packed(layer, H.dev(codecs.pack_nibbles(codes)), H.dev(e))


@pytest.mark.parametrize("m,n,k", [(1, 96, 256), (16, 2048, 7168), (16, 7168, 2048), (37, 200, 640),
                                   (64, 512, 1024), (200, 272, 512), (300, 1040, 2048), (512, 2048, 7168)])
def test_mxfp4_int8_parity(qdg, m, n, k):
    codes, e = _weights(n, k, salt=m)
    a = synth.activations_bf16_bits(m, k, workload_id=2, salt=m + 1)
    qa, sa = quant.quantize_act_int8(a)
    y64 = ref.gemm_mxfp4_int8(qa, sa, codes, e)
    for otype in (q.QDG_O_F32, q.QDG_O_BF16):
        layer, pk = _packed(n, k, codes, e, otype)
        y, plan = H.gemm(layer, pk, H.dev(qa), m, a_scales=H.dev(sa))
        # the streaming family below 64 rows, the 8-bit LDS-tiled one from 64
        assert ("family=qtile " if m >= 64 else "family=stream ") in q.qdg_plan_describe(plan, m)
        err = metrics.rel_frob(H.to_f64(y), y64)
        print(f"MXFP4xINT8 M={m} N={n} K={k} otype={otype}: rel_frob={err:.3e}")
        assert err <= (1e-3 if otype == q.QDG_O_F32 else 2e-3), err


@pytest.mark.parametrize("m", [16, 64, 128])
def test_mxfp4_int8_one_hot_extreme_codes(qdg, m):
    # a single code per row at a different k per row, unit token scale: each
    # output row is code * (dequantized weights) at that k, exact in fp32;
    # over the calls every int8 code -128 .. 127 appears (the hi/lo split of
    # -128 is -8 * 16 + 0, of 127 is 7 * 16 + 15)
    k, n = 384, 80
    codes, e = _weights(n, k, salt=7)
    w64 = ref.dequant_mxfp4(codes, e)
    vals = np.arange(-128, 128)
    layer, pk = _packed(n, k, codes, e, q.QDG_O_F32)
    seen = set()
    for base in range(0, k, m):
        ks = np.arange(base, base + m) % k
        qa = np.zeros((m, k), np.int8)
        v = vals[(np.arange(m) + base) % len(vals)]
        seen.update(v[: min(m, k - base)].tolist())
        qa[np.arange(m), ks] = v
        y = H.gemm(layer, pk, H.dev(qa), m, a_scales=H.dev(np.ones(m, np.float32)))[0]
        want = v[:, None].astype(np.float64) * w64[:, ks].T
        assert np.array_equal(H.to_f64(y)[: min(m, k - base)], want[: min(m, k - base)])
    assert seen == set(range(-128, 128))


def test_mxfp4_int8_device_quantizer_pipeline(qdg):
    # bf16 activations quantized on the device (bit-exact int8 codes and
    # scales), then the GEMM, against the oracle on the oracle's codes
    m, n, k = 48, 1024, 2048
    codes, e = _weights(n, k, salt=11)
    a = synth.activations_bf16_bits(m, k, workload_id=2, salt=12)
    qa, sa = quant.quantize_act_int8(a)
    layer, pk = _packed(n, k, codes, e, q.QDG_O_BF16)
    qa_d = torch.empty((m, k), dtype=torch.int8, device="cuda")
    sa_d = torch.empty(m, dtype=torch.float32, device="cuda")
    q.qdg_quantize_act(layer, H.bf16_dev(a).data_ptr(), m, qa_d.data_ptr(), sa_d.data_ptr(), q.current_stream())
    y, _ = H.gemm(layer, pk, qa_d, m, a_scales=sa_d)
    assert np.array_equal(qa_d.cpu().numpy(), qa)
    assert metrics.rel_frob(H.to_f64(y), ref.gemm_mxfp4_int8(qa, sa, codes, e)) <= 2e-3


@pytest.mark.parametrize("bm", [16, 32, 64, 128])
def test_mxfp4_int8_moe(qdg, bm):
    # grouped MoE: E=4 experts, top-2, gate+up over token rows and down over
    # pair rows, fp32 output against the per-pair oracle rows
    E, top_k, t, hid, n = 4, 2, 70, 512, 192
    ids, _ = ref.route_topk(synth.router_logits(t, E, salt=bm), top_k)
    ws = [_weights(n, hid, salt=100 + e) for e in range(E)]
    layer = q.layer_mxfp4_int8(n, hid, otype=q.QDG_O_F32, num_experts=E)
    pk = H.Packed(layer, H.dev(np.stack([codecs.pack_nibbles(c) for c, _ in ws])),
                  H.dev(np.stack([e for _, e in ws])))
    for per_pair in (0, 1):
        rows = t * top_k if per_pair else t
        a = synth.activations_bf16_bits(rows, hid, workload_id=2, salt=bm + per_pair)
        qa, sa = quant.quantize_act_int8(a)
        cap = q.qdg_moe_align_capacity(t, top_k, E, bm)
        sid = torch.empty(cap, dtype=torch.int32, device="cuda")
        blk = torch.empty(cap // bm, dtype=torch.int32, device="cuda")
        npad = torch.zeros(1, dtype=torch.int32, device="cuda")
        q.qdg_moe_align(H.dev(ids.astype(np.int32)).data_ptr(), t, top_k, E, bm, sid.data_ptr(), blk.data_ptr(),
                        npad.data_ptr(), q.current_stream())
        plan = q.qdg_plan_create(layer, q.moe(top_k))
        assert ("family=qtile " if bm >= 64 else "family=stream ") in q.qdg_moe_describe(plan, t, bm)
        wsp, nbytes = H.workspace(plan, t)
        y = H.out_tensor(t * top_k, n, q.QDG_O_F32)
        qa_d, sa_d = H.dev(qa), H.dev(sa)
        q.qdg_moe_gemm(plan, qa_d.data_ptr(), sa_d.data_ptr(), pk.buf.data_ptr(), sid.data_ptr(), blk.data_ptr(),
                       npad.data_ptr(), t, bm, per_pair, y.data_ptr(), wsp.data_ptr(), nbytes, q.current_stream())
        torch.cuda.synchronize()
        y64, _ = ref.moe_rows(ids, per_pair, lambda e, r: ref.gemm_mxfp4_int8(qa[r], sa[r], *ws[e]))
        assert not torch.isnan(y).any()
        err = metrics.rel_frob(H.to_f64(y), y64)
        print(f"MXFP4xINT8 MoE bm={bm} per_pair={per_pair}: rel_frob={err:.3e}")
        assert err <= 1e-3, err
