"""W4A16-NVFP4 (bf16 activations; E2M1 weights with an E4M3 scale per 16 K
and an fp32 scale per tensor) against the oracle: relative Frobenius
<= 2e-3 with bf16 output and <= 5e-5 with fp32 output (the scaled weights
are exact in bf16, the MFMA accumulates in fp32, the tensor scale is one
fp32 multiply); one-hot activations return every dequantized weight."""

import numpy as np
import pytest
import torch

import quantized_dequant_gemm_amd as q
import synth
from oracle import codecs, metrics, quant, ref
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _std(codes, sc, ts):
    return H.dev(codecs.pack_nibbles(codes)), H.dev(sc), H.dev(np.atleast_1d(np.asarray(ts, np.float32)))


def _case(n, k, otype, salt):
    codes, sc, ts = quant.quantize_nvfp4(synth.weights_f32(n, k, workload_id=10, salt=salt))
    layer = q.layer_nvfp4(n, k, otype=otype)
    qw, s, t = _std(codes, sc, ts)
    pk = H.Packed(layer, qw, s, tensor_scale=t)
    return layer, pk, codes, sc, ts


@pytest.mark.parametrize("m,n,k", [(1, 48, 256), (16, 512, 1024), (33, 130, 640), (64, 96, 1152), (100, 272, 512),
                                   (300, 200, 384)])
@pytest.mark.parametrize("otype", [q.QDG_O_F32, q.QDG_O_BF16])
def test_nvfp4_gemm(qdg, m, n, k, otype):
    layer, pk, codes, sc, ts = _case(n, k, otype, salt=m + n)
    a = synth.activations_bf16_bits(m, k, workload_id=10, salt=m)
    y64 = ref.gemm_nvfp4a16(a, codes, sc, ts)
    plan = q.qdg_plan_create(layer, q.dense())
    d = q.qdg_plan_describe(plan, m)
    fam = "family=stream" if m <= 32 else "family=tile"  # LDS-tiled family from M = 33
    assert "w4a16-nvfp4" in d and fam in d
    y, _ = H.gemm(layer, pk, H.bf16_dev(a), m)
    assert not torch.isnan(y.float()).any()
    err = metrics.rel_frob(H.to_f64(y), y64)
    print(f"NVFP4 M={m} N={n} K={k} otype={otype}: rel_frob={err:.3e}")
    assert err <= (5e-5 if otype == q.QDG_O_F32 else 2e-3), err


def test_nvfp4_one_hot_recovers_dequantized_weights(qdg):
    k, n = 256, 80
    layer, pk, codes, sc, ts = _case(n, k, q.QDG_O_F32, salt=3)
    eye = codecs.f32_to_bf16_bits(np.eye(k, dtype=np.float32))
    y, _ = H.gemm(layer, pk, H.bf16_dev(eye), k)
    want = ref.dequant_nvfp4(codes, sc, ts).T.astype(np.float32).astype(np.float64)
    assert np.array_equal(H.to_f64(y), want)


def test_nvfp4_every_code_and_scale_pattern(qdg):
    # every E2M1 code in every 16-block position, block scales over the whole
    # E4M3 range (subnormal to 448, both signs) and a non-power-of-two tensor
    # scale; the NaN scale codes 0x7F / 0xFF act as +-448 (0x7E / 0xFE)
    rng = np.random.default_rng(21)
    n, k, m = 64, 512, 24
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    codes[:16, :16] = (np.arange(16)[:, None] + np.arange(16)[None, :]) % 16
    sc = rng.integers(0, 256, (n, k // 16)).astype(np.uint8)
    sc[(sc & 0x7F) == 0x7F] -= 1
    ts = np.float32(0.0123)
    a = synth.activations_bf16_bits(m, k, workload_id=10, salt=22)
    layer = q.layer_nvfp4(n, k, otype=q.QDG_O_F32)
    y64 = ref.gemm_nvfp4a16(a, codes, sc, ts)
    qw, s, t = _std(codes, sc, ts)
    y, _ = H.gemm(layer, H.Packed(layer, qw, s, tensor_scale=t), H.bf16_dev(a), m)
    assert metrics.rel_frob(H.to_f64(y), y64) <= 5e-5
    nan_sc = sc.copy()
    nan_sc[:, 0] = np.where(nan_sc[:, 0] & 0x80, 0xFF, 0x7F)
    sc448 = sc.copy()
    sc448[:, 0] = np.where(sc448[:, 0] & 0x80, 0xFE, 0x7E)
    y_nan, _ = H.gemm(layer, H.Packed(layer, qw, H.dev(nan_sc), tensor_scale=t), H.bf16_dev(a), m)
    y_448, _ = H.gemm(layer, H.Packed(layer, qw, H.dev(sc448), tensor_scale=t), H.bf16_dev(a), m)
    assert torch.equal(y_nan, y_448)
    assert metrics.rel_frob(H.to_f64(y_448), ref.gemm_nvfp4a16(a, codes, sc448, ts)) <= 5e-5


@pytest.mark.parametrize("m,n,k,split", [(129, 200, 640, 0), (300, 520, 1280, 3), (1024, 2048, 4096, 0),
                                         (64, 4096, 2048, 0)])
@pytest.mark.parametrize("otype", [q.QDG_O_F32, q.QDG_O_BF16])
def test_nvfp4_tiled(qdg, m, n, k, split, otype):
    # the LDS-tiled family: ragged M (partial 128-row blocks), ragged N (a
    # partial 256-column block), K split heuristically or pinned
    layer, pk, codes, sc, ts = _case(n, k, otype, salt=m + 2 * n)
    a = synth.activations_bf16_bits(m, k, workload_id=10, salt=m + 1)
    t = q.TuningConfig(block_m=128, split_k=split)
    y, plan = H.gemm(layer, pk, H.bf16_dev(a), m, tuning=t)
    d = q.qdg_plan_describe(plan, m)
    assert "family=tile" in d and "32x32x16_bf16" in d and (not split or f"split_k={split}" in d), d
    assert not torch.isnan(y.float()).any()
    err = metrics.rel_frob(H.to_f64(y), ref.gemm_nvfp4a16(a, codes, sc, ts))
    print(f"NVFP4 tiled M={m} N={n} K={k} split={split} otype={otype}: rel_frob={err:.3e}")
    assert err <= (5e-5 if otype == q.QDG_O_F32 else 2e-3), err


@pytest.mark.parametrize("split", [2, 3])
def test_nvfp4_split_k(qdg, split):
    m, n, k = 20, 160, 1536
    layer, pk, codes, sc, ts = _case(n, k, q.QDG_O_F32, salt=40 + split)
    a = synth.activations_bf16_bits(m, k, workload_id=10, salt=40 + split)
    t = q.TuningConfig(block_m=32, block_n=32, waves=4, split_k=split)
    y, plan = H.gemm(layer, pk, H.bf16_dev(a), m, tuning=t)
    assert f"split_k={split}" in q.qdg_plan_describe(plan, m)
    assert metrics.rel_frob(H.to_f64(y), ref.gemm_nvfp4a16(a, codes, sc, ts)) <= 5e-5


def test_nvfp4_decode_layer_shape(qdg):
    # the dense up-projection shape at M = 16, as the benchmark runs it
    m, n, k = 16, 14336, 4096
    layer, pk, codes, sc, ts = _case(n, k, q.QDG_O_BF16, salt=5)
    a = synth.activations_bf16_bits(m, k, workload_id=10, salt=6)
    y, _ = H.gemm(layer, pk, H.bf16_dev(a), m)
    err = metrics.rel_frob(H.to_f64(y), ref.gemm_nvfp4a16(a, codes, sc, ts))
    print(f"NVFP4 M={m} N={n} K={k}: rel_frob={err:.3e}")
    assert err <= 2e-3, err


# The larger cases give every expert several blocks (about 200 pairs each),
# two N blocks of the 256-column tiles (the second partly filled) and eight K
# groups, so the tiled instance runs its steady-state copy ring.
@pytest.mark.parametrize("per_pair,bm,t,n,k", [(0, 16, 40, 96, 256), (1, 32, 40, 96, 256), (0, 128, 40, 96, 256),
                                               (1, 128, 40, 96, 256), (0, 128, 400, 384, 1024),
                                               (1, 128, 400, 384, 1024), (1, 64, 400, 384, 1024)])
def test_nvfp4_moe(qdg, per_pair, bm, t, n, k):
    E, top_k = 4, 2
    ids, _ = ref.route_topk(synth.router_logits(t, E, salt=5 + per_pair), top_k)
    qs = [quant.quantize_nvfp4(synth.weights_f32(n, k, workload_id=10, salt=700 + e)) for e in range(E)]
    rows_in = t * top_k if per_pair else t
    a = synth.activations_bf16_bits(rows_in, k, workload_id=10, salt=77 + per_pair)
    y64, _ = ref.moe_rows(ids, per_pair, lambda e, rows: ref.gemm_nvfp4a16(a[rows], *qs[e]))
    layer = q.layer_nvfp4(n, k, otype=q.QDG_O_F32, num_experts=E)
    pk = H.Packed(layer, H.dev(np.stack([codecs.pack_nibbles(c) for c, _, _ in qs])),
                  H.dev(np.stack([s for _, s, _ in qs])), tensor_scale=H.dev(np.array([x for _, _, x in qs], np.float32)))
    cap = q.qdg_moe_align_capacity(t, top_k, E, bm)
    sid = torch.empty(cap, dtype=torch.int32, device="cuda")
    blk = torch.empty(cap // bm, dtype=torch.int32, device="cuda")
    npad = torch.zeros(1, dtype=torch.int32, device="cuda")
    ids_dev = H.dev(ids.astype(np.int32))
    q.qdg_moe_align(ids_dev.data_ptr(), t, top_k, E, bm, sid.data_ptr(), blk.data_ptr(), npad.data_ptr(),
                    q.current_stream())
    plan = q.qdg_plan_create(layer, q.moe(top_k))
    assert "w4a16-nvfp4" in q.qdg_moe_describe(plan, t, bm)
    wsb = q.qdg_plan_workspace(plan, t)
    wsp = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
    a_dev = H.bf16_dev(a)
    y = H.out_tensor(t * top_k, n, q.QDG_O_F32)
    q.qdg_moe_gemm(plan, a_dev.data_ptr(), None, pk.buf.data_ptr(), sid.data_ptr(), blk.data_ptr(), npad.data_ptr(),
                   t, bm, per_pair, y.data_ptr(), wsp.data_ptr(), wsb, q.current_stream())
    torch.cuda.synchronize()
    assert not torch.isnan(y).any()
    assert metrics.rel_frob(H.to_f64(y), y64) <= 5e-5


@pytest.mark.parametrize("n,k,e", [(200, 512, 1), (64, 256, 3)])
def test_nvfp4_device_quantizer_matches_oracle(qdg, n, k, e):
    # the library's NVFP4 producer takes the same binary32 decisions as the
    # oracle's quantizer: codes, block scales and tensor scales bit for bit
    w = np.stack([synth.weights_f32(n, k, workload_id=10, salt=900 + i) for i in range(e)])
    if e > 1:
        w[1] = 0.0  # an all-zero expert: tensor scale 1, zero codes and scales
    layer = q.layer_nvfp4(n, k, num_experts=e)
    qw = torch.empty((e, n, k // 2), dtype=torch.uint8, device="cuda")
    sc = torch.empty((e, n, k // 16), dtype=torch.uint8, device="cuda")
    ts = torch.empty(e, dtype=torch.float32, device="cuda")
    w_dev = H.dev(w)
    q.qdg_quantize_weights(layer, w_dev.data_ptr(), qw.data_ptr(), sc.data_ptr(), ts.data_ptr(), q.current_stream())
    torch.cuda.synchronize()
    for i in range(e):
        codes, s, t = quant.quantize_nvfp4(w[i])
        assert ts[i].item() == float(t)
        assert np.array_equal(sc[i].cpu().numpy(), s)
        assert np.array_equal(qw[i].cpu().numpy(), codecs.pack_nibbles(codes))
