"""W8A16 (bf16 activations, int8 weights with fp32 per-channel scales)
against the oracle: relative Frobenius <= 2e-3 with bf16 output and <= 5e-5
with fp32 output (the MFMA sums of A * q are exact products accumulated in
fp32, the scale is one fp32 multiply); one-hot activations return every
dequantized weight q * s exactly."""

import numpy as np
import pytest
import torch

import quantized_dequant_gemm_amd as q
import synth
from oracle import codecs, metrics, quant, ref
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _case(n, k, otype, salt):
    w = synth.weights_f32(n, k, workload_id=9, salt=salt)
    qw, sw = quant.quantize_int8_per_channel(w)
    layer = q.layer_w8a16(n, k, otype=otype)
    pk = H.Packed(layer, H.dev(qw.astype(np.int8)), H.dev(sw))
    return layer, pk, qw, sw


@pytest.mark.parametrize("m,n,k", [(1, 48, 256), (16, 512, 1024), (33, 130, 640), (64, 96, 1152), (100, 272, 512),
                                   (300, 200, 384)])
@pytest.mark.parametrize("otype", [q.QDG_O_F32, q.QDG_O_BF16])
def test_w8a16_gemm(qdg, m, n, k, otype):
    layer, pk, qw, sw = _case(n, k, otype, salt=m + n)
    a = synth.activations_bf16_bits(m, k, workload_id=9, salt=m)
    y64 = ref.gemm_w8a16(a, qw, sw)
    plan = q.qdg_plan_create(layer, q.dense())
    d = q.qdg_plan_describe(plan, m)
    fam = "family=stream" if m <= 32 else "family=tile"  # LDS-tiled family from M = 33
    assert "w8a16-int8" in d and fam in d
    y, _ = H.gemm(layer, pk, H.bf16_dev(a), m)
    assert not torch.isnan(y.float()).any()
    err = metrics.rel_frob(H.to_f64(y), y64)
    assert err <= (5e-5 if otype == q.QDG_O_F32 else 2e-3), err


def test_w8a16_one_hot_recovers_dequantized_weights(qdg):
    k, n = 384, 80
    layer, pk, qw, sw = _case(n, k, q.QDG_O_F32, salt=3)
    eye = codecs.f32_to_bf16_bits(np.eye(k, dtype=np.float32))
    y, _ = H.gemm(layer, pk, H.bf16_dev(eye), k)
    want = (qw.astype(np.float64) * sw.astype(np.float64)[:, None]).T
    assert np.array_equal(H.to_f64(y), want.astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("m,n,k,split", [(129, 200, 640, 0), (300, 520, 1280, 3), (1024, 2048, 4096, 0),
                                         (64, 4096, 2048, 0)])
@pytest.mark.parametrize("otype", [q.QDG_O_F32, q.QDG_O_BF16])
def test_w8a16_tiled(qdg, m, n, k, split, otype):
    # the LDS-tiled family: ragged M (partial 128-row blocks), ragged N (a
    # partial 256-column block), K split heuristically or pinned
    layer, pk, qw, sw = _case(n, k, otype, salt=m + 2 * n)
    a = synth.activations_bf16_bits(m, k, workload_id=9, salt=m + 1)
    t = q.TuningConfig(block_m=128, split_k=split)
    y, plan = H.gemm(layer, pk, H.bf16_dev(a), m, tuning=t)
    d = q.qdg_plan_describe(plan, m)
    assert "family=tile" in d and "32x32x16_bf16" in d and (not split or f"split_k={split}" in d), d
    assert not torch.isnan(y.float()).any()
    err = metrics.rel_frob(H.to_f64(y), ref.gemm_w8a16(a, qw, sw))
    print(f"W8A16 tiled M={m} N={n} K={k} split={split} otype={otype}: rel_frob={err:.3e}")
    assert err <= (5e-5 if otype == q.QDG_O_F32 else 2e-3), err


@pytest.mark.parametrize("split", [2, 3])
def test_w8a16_split_k(qdg, split):
    m, n, k = 20, 160, 1536
    layer, pk, qw, sw = _case(n, k, q.QDG_O_F32, salt=40 + split)
    a = synth.activations_bf16_bits(m, k, workload_id=9, salt=40 + split)
    t = q.TuningConfig(block_m=32, block_n=32, waves=4, split_k=split)
    y, plan = H.gemm(layer, pk, H.bf16_dev(a), m, tuning=t)
    assert f"split_k={split}" in q.qdg_plan_describe(plan, m)
    assert metrics.rel_frob(H.to_f64(y), ref.gemm_w8a16(a, qw, sw)) <= 5e-5


# The larger cases give every expert several blocks (about 200 pairs each),
# two N blocks of the 256-column tiles (the second partly filled) and eight K
# groups, so the tiled instance runs its steady-state copy ring.
@pytest.mark.parametrize("bm,t,n,k", [(16, 40, 96, 256), (128, 40, 96, 256), (128, 400, 384, 1024),
                                      (32, 400, 384, 1024)])
def test_w8a16_moe(qdg, bm, t, n, k):
    E, top_k = 4, 2
    ids, _ = ref.route_topk(synth.router_logits(t, E, salt=5), top_k)
    qs = [quant.quantize_int8_per_channel(synth.weights_f32(n, k, workload_id=9, salt=700 + e)) for e in range(E)]
    a = synth.activations_bf16_bits(t, k, workload_id=9, salt=77)
    y64, _ = ref.moe_rows(ids, 0, lambda e, rows: ref.gemm_w8a16(a[rows], qs[e][0], qs[e][1]))
    layer = q.layer_w8a16(n, k, otype=q.QDG_O_F32, num_experts=E)
    pk = H.Packed(layer, H.dev(np.stack([x.astype(np.int8) for x, _ in qs])), H.dev(np.stack([s for _, s in qs])))
    cap = q.qdg_moe_align_capacity(t, top_k, E, bm)
    sid = torch.empty(cap, dtype=torch.int32, device="cuda")
    blk = torch.empty(cap // bm, dtype=torch.int32, device="cuda")
    npad = torch.zeros(1, dtype=torch.int32, device="cuda")
    ids_dev = H.dev(ids.astype(np.int32))
    q.qdg_moe_align(ids_dev.data_ptr(), t, top_k, E, bm, sid.data_ptr(), blk.data_ptr(), npad.data_ptr(),
                    q.current_stream())
    plan = q.qdg_plan_create(layer, q.moe(top_k))
    wsb = q.qdg_plan_workspace(plan, t)
    wsp = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
    a_dev = H.bf16_dev(a)
    y = H.out_tensor(t * top_k, n, q.QDG_O_F32)
    q.qdg_moe_gemm(plan, a_dev.data_ptr(), None, pk.buf.data_ptr(), sid.data_ptr(), blk.data_ptr(), npad.data_ptr(),
                   t, bm, 0, y.data_ptr(), wsp.data_ptr(), wsb, q.current_stream())
    torch.cuda.synchronize()
    assert not torch.isnan(y).any()
    assert metrics.rel_frob(H.to_f64(y), y64) <= 5e-5
