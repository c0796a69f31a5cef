"""Grouped MoE W4A16 parity: the expert sort (bit-exact) and the grouped GEMM
(relative Frobenius <= 2e-3 with bf16 output, every real pair row written,
nothing else touched)."""

import numpy as np
import pytest
import torch

import quantized_dequant_gemm_amd as q
import synth
from oracle import codecs, metrics, quant, ref
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _align_dev(ids, E, bm):
    t, top_k = ids.shape
    cap = q.qdg_moe_align_capacity(t, top_k, E, bm)
    sid = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
    blk = torch.full((cap // bm,), -7, dtype=torch.int32, device="cuda")
    npad = torch.zeros(1, dtype=torch.int32, device="cuda")
    q.qdg_moe_align(H.dev(ids.astype(np.int32)).data_ptr(), t, top_k, E, bm, sid.data_ptr(), blk.data_ptr(),
                    npad.data_ptr(), q.current_stream())
    torch.cuda.synchronize()
    return sid, blk, npad, cap


@pytest.mark.parametrize("t", [1, 64, 512, 4096])
@pytest.mark.parametrize("bm", [16, 32, 64, 128])
def test_moe_align_bit_exact(qdg, t, bm):
    ids, _ = ref.route_topk(synth.router_logits(t, 256, salt=t), 8)
    sid, blk, npad, cap = _align_dev(ids, 256, bm)
    r_sid, r_blk, r_np = ref.moe_align(ids, 256, bm)
    n = int(npad.item())
    assert n == r_np
    s = sid.cpu().numpy()
    b = blk.cpu().numpy()
    assert np.array_equal(s[:n], r_sid)
    assert np.all(s[n:] == t * 8)              # sentinel past the end
    assert np.array_equal(b[:n // bm], r_blk)
    assert np.all(b[n // bm:] == -1)


def _experts(E, n, k, salt):
    qs, ss = [], []
    for e in range(E):
        w = synth.weights_f32(n, k, workload_id=4, salt=1000 * salt + e)
        qv, s = quant.quantize_int4_sym(w)
        qs.append(qv)
        ss.append(s)
    return qs, ss


def _moe_packed(qs, ss, n, k):
    E = len(qs)
    layer = q.layer_w4a16(n, k, num_experts=E)
    qw = H.dev(np.stack([codecs.pack_nibbles(codecs.encode_int4(x)) for x in qs]))
    sc = H.dev(np.stack(ss).view(np.int16))
    return layer, H.Packed(layer, qw, sc)


def _moe_gemm(layer, pk, a_dev, ids, bm, a_per_pair, top_k, tuning=None, batch_invariant=0):
    t = ids.shape[0]
    sid, blk, npad, cap = _align_dev(ids, layer.num_experts, bm)
    plan = q.qdg_plan_create(layer, q.moe(top_k, batch_invariant=batch_invariant), tuning)
    ws, nbytes = H.workspace(plan, t)
    y = H.out_tensor(t * top_k, layer.n, q.QDG_O_BF16)
    q.qdg_moe_gemm(plan, a_dev.data_ptr(), None, pk.buf.data_ptr(), sid.data_ptr(), blk.data_ptr(),
                   npad.data_ptr(), t, bm, a_per_pair, y.data_ptr(), ws.data_ptr(), nbytes, q.current_stream())
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("t,bm", [(8, 16), (64, 16), (256, 32), (300, 64), (300, 128), (1024, 128)])
def test_moe_gemm_small_experts(qdg, t, bm):
    # E=16 experts, top-4, hidden 1024 -> intermediate 2*256 (gate+up) and back
    E, top_k, hid, inter = 16, 4, 1024, 256
    ids, _ = ref.route_topk(synth.router_logits(t, E, salt=t), top_k)
    qs, ss = _experts(E, 2 * inter, hid, salt=1)
    layer, pk = _moe_packed(qs, ss, 2 * inter, hid)
    x = synth.activations_bf16_bits(t, hid, workload_id=4, salt=t)
    y = _moe_gemm(layer, pk, H.bf16_dev(x), ids, bm, 0, top_k)
    y64 = ref.moe_gemm_rows(x, ids, lambda e: ref.dequant_int4_sym(qs[e], ss[e]), input_is_per_pair=False)
    assert metrics.rel_frob(H.to_f64(y), y64) <= 2e-3
    # down projection: one input row per pair
    qd, sd = _experts(E, hid, inter, salt=2)
    layer_d, pk_d = _moe_packed(qd, sd, hid, inter)
    h = synth.moe_hidden_bf16_bits(t * top_k, inter, salt=t)
    yd = _moe_gemm(layer_d, pk_d, H.bf16_dev(h), ids, bm, 1, top_k)
    yd64 = ref.moe_gemm_rows(h, ids, lambda e: ref.dequant_int4_sym(qd[e], sd[e]), input_is_per_pair=True)
    assert metrics.rel_frob(H.to_f64(yd), yd64) <= 2e-3


@pytest.mark.parametrize("bm,pin_ws", [(16, False), (16, True), (32, False), (128, False)])
def test_moe_single_expert_equals_dense(qdg, bm, pin_ws):
    # everything routed to expert 0 of 2: the MoE blocks hold the same rows as
    # the dense GEMM run block by block with the same kernel family, so every
    # output matches bitwise (16-row blocks with this short K: streaming, or
    # weight streaming when a tuning pins it; 32: the batch-invariant plan's
    # streaming blocks; 128: LDS-tiled)
    t, hid, n = 40, 512, 128
    qs, ss = _experts(2, n, hid, salt=3)
    layer, pk = _moe_packed(qs, ss, n, hid)
    x = synth.activations_bf16_bits(t, hid, workload_id=4, salt=5)
    ids = np.zeros((t, 1), np.int32)
    tm = q.TuningConfig(block_n=64, waves=8) if pin_ws else None
    plan = q.qdg_plan_create(layer, q.moe(1, batch_invariant=int(bm == 32)), tm)
    fam = q.qdg_moe_describe(plan, t, bm).split("family=")[1].split()[0]
    assert fam == {16: "wstream" if pin_ws else "stream", 32: "stream", 128: "tile"}[bm]
    y = _moe_gemm(layer, pk, H.bf16_dev(x), ids, bm, 0, 1, tuning=tm, batch_invariant=int(bm == 32))
    if bm == 16 and pin_ws:
        t1 = q.TuningConfig(block_m=16, block_n=64, split_k=1)
        yd = torch.cat([H.w4a16(x[r:r + 16], qs[0], ss[0], None, tuning=t1) for r in range(0, t, 16)])
    elif bm == 16:
        t1 = q.TuningConfig(block_m=16, block_n=64, waves=4, split_k=1)
        yd = H.w4a16(x, qs[0], ss[0], None, tuning=t1)
    elif bm == 32:
        t1 = q.TuningConfig(block_m=bm, block_n=32, split_k=1)
        yd = H.w4a16(x, qs[0], ss[0], None, tuning=t1)
    else:
        t1 = q.TuningConfig(block_m=128, split_k=1)
        yd = H.w4a16(x, qs[0], ss[0], None, tuning=t1)
    assert torch.equal(y, yd)


@pytest.mark.parametrize("proj,t,bm", [("gate_up", 64, 16), ("gate_up", 512, 128), ("gate_up", 4096, 128), ("gate_up", 4096, 64),
                                       ("down", 64, 16), ("down", 512, 32), ("down", 4096, 128)])
def test_moe_full_size_sampled_rows(qdg, proj, t, bm):
    # the real MoE shapes (E=256, top-8, hidden 7168, intermediate 2048):
    # gate+up K=7168 -> N=4096 over token rows, down K=2048 -> N=7168 over
    # pair rows; expert weights are quantized on the device, outputs checked
    # on sampled pairs
    E, top_k, hid, inter = 256, 8, 7168, 2048
    n, k = (2 * inter, hid) if proj == "gate_up" else (hid, inter)
    per_pair = proj == "down"
    layer = q.layer_w4a16(n, k, num_experts=E)
    qw = torch.empty((E, n, k // 2), dtype=torch.uint8, device="cuda")
    sc = torch.empty((E, n, k // 128), dtype=torch.int16, device="cuda")
    ids, _ = ref.route_topk(synth.router_logits(t, E), top_k)
    pairs = sorted({0, 7, 100, 257, t * top_k // 2 + 3, t * top_k - 1})
    sample_experts = sorted({int(ids.reshape(-1)[p]) for p in pairs})
    w_host = {}
    for e in range(E):
        w = synth.device_normal_f32((n, k), 0.02, seed=synth.seed_for(4, synth.TID_W, e + (E if per_pair else 0)))
        if e in sample_experts:
            w_host[e] = w.cpu().numpy()
        q.qdg_quantize_weights(q.layer_w4a16(n, k), w.data_ptr(), qw[e].data_ptr(), sc[e].data_ptr(), None,
                               q.current_stream())
        del w
    pk = H.Packed(layer, qw, sc)
    del qw, sc
    if per_pair:
        x = synth.moe_hidden_bf16_bits(t * top_k, k, salt=t)
    else:
        x = synth.activations_bf16_bits(t, k, workload_id=4)
    y = _moe_gemm(layer, pk, H.bf16_dev(x), ids, bm, 1 if per_pair else 0, top_k)
    fam = q.qdg_moe_describe(q.qdg_plan_create(layer, q.moe(top_k)), t, bm).split("family=")[1].split()[0]
    assert fam == ("tile" if bm in (32, 64, 128) else "stream")
    xf = codecs.bf16_bits_to_f64(x)
    for p in pairs:
        e = int(ids.reshape(-1)[p])
        qv, s = quant.quantize_int4_sym(w_host[e])
        yr = xf[p if per_pair else p // top_k] @ ref.dequant_int4_sym(qv, s).T
        err = metrics.rel_frob(H.to_f64(y[p]), yr)
        print(f"MoE {proj} T={t} bm={bm} pair {p} expert {e}: rel_frob={err:.3e}")
        assert err <= 2e-3, (p, err)
    # every real pair row was written (the output was prefilled with NaN)
    assert not torch.isnan(y.float()).any()


@pytest.mark.parametrize("t,bm,inter", [(8, 16, 256), (64, 16, 144), (64, 32, 256), (64, 32, 144), (300, 64, 256),
                                         (300, 64, 144), (300, 128, 256), (1024, 128, 144)])
@pytest.mark.parametrize("otype", [q.QDG_O_F32, q.QDG_O_BF16])
def test_moe_gate_up_silu_mul_epilogue(qdg, t, bm, inter, otype):
    # fused gate+up (n = 2I) with the SiLU*mul epilogue: Y = silu(G) * U,
    # [T*top_k][I]; 16-row blocks run the streaming family (four tiles, two
    # gate + two up, per workgroup), 32-, 64- and 128-row blocks the LDS-tiled
    # one (I = 144: an odd number of gate tiles, so a workgroup's tile slots
    # run partly past the layer)
    E, top_k, hid = 16, 4, 1024
    ids, _ = ref.route_topk(synth.router_logits(t, E, salt=t + 11), top_k)
    qs, ss = _experts(E, 2 * inter, hid, salt=9)
    layer = q.layer_w4a16(2 * inter, hid, num_experts=E, otype=otype)
    qw = H.dev(np.stack([codecs.pack_nibbles(codecs.encode_int4(x)) for x in qs]))
    sc = H.dev(np.stack(ss).view(np.int16))
    pk = H.Packed(layer, qw, sc)
    x = synth.activations_bf16_bits(t, hid, workload_id=4, salt=t + 12)
    a_dev = H.bf16_dev(x)
    sid, blk, npad, cap = _align_dev(ids, E, bm)
    plan = q.qdg_plan_create(layer, q.moe(top_k, epilogue=q.QDG_EPI_SILU_MUL))
    desc = q.qdg_moe_describe(plan, t, bm)
    assert "epilogue=silu_mul" in desc and ("family=tile" in desc) == (bm in (32, 64, 128))
    ws, nbytes = H.workspace(plan, t)
    y = H.out_tensor(t * top_k, inter, otype)
    q.qdg_moe_gemm(plan, a_dev.data_ptr(), None, pk.buf.data_ptr(), sid.data_ptr(), blk.data_ptr(),
                   npad.data_ptr(), t, bm, 0, y.data_ptr(), ws.data_ptr(), nbytes, q.current_stream())
    torch.cuda.synchronize()
    gu64 = ref.moe_gemm_rows(x, ids, lambda e: ref.dequant_int4_sym(qs[e], ss[e]), input_is_per_pair=False)
    h64 = ref.silu_mul(gu64)
    assert not torch.isnan(y.float()).any()
    err = metrics.rel_frob(H.to_f64(y), h64)
    print(f"silu*mul T={t} bm={bm} otype={otype}: rel_frob={err:.3e}")
    assert err <= (1e-3 if otype == q.QDG_O_F32 else 2e-3), err


@pytest.mark.parametrize("t,otype", [(64, q.QDG_O_F32), (64, q.QDG_O_BF16), (1000, q.QDG_O_BF16)])
def test_moe_combine(qdg, t, otype):
    top_k, n = 8, 7168
    r = np.random.default_rng(40 + t)
    y = r.normal(size=(t * top_k, n)).astype(np.float32)
    w = r.uniform(0.0, 0.5, t * top_k).astype(np.float32)
    y_dev, w_dev = H.dev(y), H.dev(w)
    out = H.out_tensor(t, n, otype)
    q.qdg_moe_combine(y_dev.data_ptr(), w_dev.data_ptr(), t, top_k, n, out.data_ptr(), otype, q.current_stream())
    out2 = H.out_tensor(t, n, otype)
    q.qdg_moe_combine(y_dev.data_ptr(), w_dev.data_ptr(), t, top_k, n, out2.data_ptr(), otype, q.current_stream())
    torch.cuda.synchronize()
    assert torch.equal(out, out2)  # fixed summation order
    ref64 = ref.moe_combine(y, w, top_k)
    err = metrics.rel_frob(H.to_f64(out), ref64)
    assert err <= (1e-6 if otype == q.QDG_O_F32 else 2e-3), err
