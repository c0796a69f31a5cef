"""W4A4 (MXFP4 weights x MXFP4 activations) against the oracle: the
activation quantizer reproduces the oracle's E2M1 codes and E8M0 scales bit
for bit, and the GEMM (streaming family, fp4 x fp4 scaled MFMAs with both
block scales applied by the hardware) matches the fp64 product of the
decoded operands: relative Frobenius <= 1e-3 with fp32 output (products are
exact, only the fp32 accumulation rounds), <= 2e-3 with bf16 output."""

import numpy as np
import pytest
import torch

import quantized_dequant_gemm_amd as q
import synth
from oracle import codecs, metrics, quant, ref
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _act_fp4_dev(a_bits, m, k):
    layer = q.layer_w4a4(16, k)
    qa = torch.empty((m, k // 2), dtype=torch.uint8, device="cuda")
    sa = torch.empty((m, k // 32), dtype=torch.uint8, device="cuda")
    q.qdg_quantize_act(layer, H.bf16_dev(a_bits).data_ptr(), m, qa.data_ptr(), sa.data_ptr(), q.current_stream())
    torch.cuda.synchronize()
    return qa, sa


@pytest.mark.parametrize("m,k", [(1, 128), (7, 384), (64, 2048)])
def test_act_mxfp4_bit_exact(qdg, m, k):
    a = synth.activations_bf16_bits(m, k, workload_id=8, salt=m)
    # plant the E2M1 tie cases and a zero block in row 0
    vals = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -0.25, -0.75, -5.0, 7.0, -0.1, 0.0], np.float32)
    a[0, :vals.size] = codecs.f32_to_bf16_bits(vals)
    if k >= 64:
        a[0, 32:64] = 0
    codes, e = quant.quantize_act_mxfp4(a)
    qa, sa = _act_fp4_dev(a, m, k)
    assert np.array_equal(sa.cpu().numpy(), e)
    assert np.array_equal(qa.cpu().numpy(), codecs.pack_nibbles(codes))


def test_act_mxfp4_every_bf16_magnitude(qdg):
    # Every bf16 value of magnitude <= 7.9375, both signs (every E2M1 tie,
    # saturation above 6, signed zeros, bf16 subnormals): each 32-block also
    # holds +-7.9375, so its shared exponent is X = floor(log2 7.9375) - 2 = 0
    # and the codes are the E2M1 encoding of the inputs themselves, bit for
    # bit as the oracle's encoder gives them.
    pos = np.arange(0, 0x40FF, dtype=np.uint16)
    vals = np.concatenate([pos, pos | np.uint16(0x8000)])
    per = 31
    nblk = -(-vals.size // per)
    nblk = -(-nblk // 8) * 8  # whole rows of 8 blocks
    grid = np.zeros((nblk, 32), dtype=np.uint16)
    grid[:, 0] = np.where(np.arange(nblk) % 2 == 0, 0x40FE, 0xC0FE)  # +-7.9375
    flat = np.zeros(nblk * per, dtype=np.uint16)
    flat[: vals.size] = vals
    grid[:, 1:] = flat.reshape(nblk, per)
    a = grid.reshape(nblk // 8, 256)
    m, k = a.shape
    codes, e = quant.quantize_act_mxfp4(a)
    assert np.all(e == 127)
    qa, sa = _act_fp4_dev(a, m, k)
    assert np.array_equal(sa.cpu().numpy(), e)
    got = qa.cpu().numpy()
    want = codecs.pack_nibbles(codes)
    bad = np.argwhere(got != want)
    assert bad.size == 0, [(hex(a[r, 2 * c]), hex(a[r, 2 * c + 1]), hex(got[r, c]), hex(want[r, c])) for r, c in bad[:8]]


def _w4a4_case(m, n, k, otype, salt):
    w = synth.weights_f32(n, k, workload_id=8, salt=salt)
    wc, we = quant.quantize_mxfp4(w)
    a = synth.activations_bf16_bits(m, k, workload_id=8, salt=salt + 1)
    ac, ae = quant.quantize_act_mxfp4(a)
    y64 = ref.gemm_w4a4(ac, ae, wc, we)
    layer = q.layer_w4a4(n, k, otype=otype)
    pk = H.Packed(layer, H.dev(codecs.pack_nibbles(wc)), H.dev(we))
    return layer, pk, H.dev(codecs.pack_nibbles(ac)), H.dev(ae), y64


@pytest.mark.parametrize("m,n,k", [(1, 48, 256), (16, 512, 1024), (40, 130, 640), (100, 272, 512), (300, 96, 384),
                                   (640, 520, 1280)])
@pytest.mark.parametrize("otype", [q.QDG_O_F32, q.QDG_O_BF16])
def test_w4a4_gemm(qdg, m, n, k, otype):
    layer, pk, qa, sa, y64 = _w4a4_case(m, n, k, otype, salt=m + n)
    plan = q.qdg_plan_create(layer, q.dense())
    fam = "family=qtile" if m > 128 else "family=stream"  # fp4 x fp4 LDS-tiled family above 128 rows
    assert "w4a4-mxfp4" in q.qdg_plan_describe(plan, m) and fam in q.qdg_plan_describe(plan, m)
    y, _ = H.gemm(layer, pk, qa, m, a_scales=sa)
    assert not torch.isnan(y.float()).any()
    err = metrics.rel_frob(H.to_f64(y), y64)
    assert err <= (1e-3 if otype == q.QDG_O_F32 else 2e-3), err


def test_w4a4_quantizer_then_gemm_end_to_end(qdg):
    # bf16 activations through the library's own quantizer, then the GEMM
    m, n, k = 24, 200, 1024
    w = synth.weights_f32(n, k, workload_id=8, salt=77)
    wc, we = quant.quantize_mxfp4(w)
    a = synth.activations_bf16_bits(m, k, workload_id=8, salt=78)
    ac, ae = quant.quantize_act_mxfp4(a)
    y64 = ref.gemm_w4a4(ac, ae, wc, we)
    layer = q.layer_w4a4(n, k, otype=q.QDG_O_F32)
    pk = H.Packed(layer, H.dev(codecs.pack_nibbles(wc)), H.dev(we))
    qa, sa = _act_fp4_dev(a, m, k)
    y, _ = H.gemm(layer, pk, qa, m, a_scales=sa)
    assert metrics.rel_frob(H.to_f64(y), y64) <= 1e-3


@pytest.mark.parametrize("t,bm,per_pair", [(8, 16, 0), (64, 32, 1), (300, 64, 0), (300, 128, 0), (600, 128, 1)])
def test_w4a4_moe(qdg, t, bm, per_pair):
    E, top_k = 8, 2
    n, k = (256, 512) if not per_pair else (512, 256)
    ids, _ = ref.route_topk(synth.router_logits(t, E, salt=t + 11), top_k)
    ws = [synth.weights_f32(n, k, workload_id=8, salt=500 + e) for e in range(E)]
    qs = [quant.quantize_mxfp4(w) for w in ws]
    rows_in = t * top_k if per_pair else t
    a = synth.activations_bf16_bits(rows_in, k, workload_id=8, salt=t)
    ac, ae = quant.quantize_act_mxfp4(a)
    y64, _ = ref.moe_rows(ids, per_pair, lambda e, rows: ref.gemm_w4a4(ac[rows], ae[rows], qs[e][0], qs[e][1]))
    layer = q.layer_w4a4(n, k, otype=q.QDG_O_F32, num_experts=E)
    pk = H.Packed(layer, H.dev(np.stack([codecs.pack_nibbles(c) for c, _ in qs])), H.dev(np.stack([x for _, x in qs])))
    cap = q.qdg_moe_align_capacity(t, top_k, E, bm)
    sid = torch.empty(cap, dtype=torch.int32, device="cuda")
    blk = torch.empty(cap // bm, dtype=torch.int32, device="cuda")
    npad = torch.zeros(1, dtype=torch.int32, device="cuda")
    ids_dev = H.dev(ids.astype(np.int32))
    q.qdg_moe_align(ids_dev.data_ptr(), t, top_k, E, bm, sid.data_ptr(), blk.data_ptr(), npad.data_ptr(),
                    q.current_stream())
    plan = q.qdg_plan_create(layer, q.moe(top_k))
    assert ("family=qtile " if bm in (64, 128) else "family=stream ") in q.qdg_moe_describe(plan, t, bm)
    wsb = q.qdg_plan_workspace(plan, t)
    wsp = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
    a_dev, s_dev = H.dev(codecs.pack_nibbles(ac)), H.dev(ae)
    y = H.out_tensor(t * top_k, n, q.QDG_O_F32)
    q.qdg_moe_gemm(plan, a_dev.data_ptr(), s_dev.data_ptr(), pk.buf.data_ptr(), sid.data_ptr(), blk.data_ptr(),
                   npad.data_ptr(), t, bm, per_pair, y.data_ptr(), wsp.data_ptr(), wsb, q.current_stream())
    torch.cuda.synchronize()
    assert not torch.isnan(y).any(), "a pair row was not written"
    assert metrics.rel_frob(H.to_f64(y), y64) <= 1e-3


@pytest.mark.parametrize("split", [1, 3])
def test_w4a4_tiled_split_k(qdg, split):
    # the LDS-tiled family with K split into fixed-order fp32 partials
    m, n, k = 200, 300, 1536
    layer, pk, qa, sa, y64 = _w4a4_case(m, n, k, q.QDG_O_F32, salt=900 + split)
    t = q.TuningConfig(block_m=128, split_k=split)
    y, plan = H.gemm(layer, pk, qa, m, a_scales=sa, tuning=t)
    d = q.qdg_plan_describe(plan, m)
    assert "family=qtile" in d and f"split_k={split}" in d
    assert metrics.rel_frob(H.to_f64(y), y64) <= 1e-3
