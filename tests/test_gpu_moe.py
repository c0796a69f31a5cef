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


@pytest.mark.parametrize("t,bm,stream", [(8, 16, False), (64, 16, False), (64, 16, True), (256, 32, False),
                                         (300, 64, False), (300, 128, False), (1024, 128, False)])
def test_moe_gemm_small_experts(qdg, t, bm, stream):
    # E=16 experts, top-4, hidden 1024 -> intermediate 2*256 (gate+up) and
    # back; 16-row blocks of these short K run 16 x 512 tiles, or the
    # streaming family when a tuning pins it
    E, top_k, hid, inter = 16, 4, 1024, 256
    tun = q.TuningConfig(block_n=64, waves=4) if stream else None
    ids, _ = ref.route_topk(synth.router_logits(t, E, salt=t), top_k)
    qs, ss = _experts(E, 2 * inter, hid, salt=1)
    layer, pk = _moe_packed(qs, ss, 2 * inter, hid)
    x = synth.activations_bf16_bits(t, hid, workload_id=4, salt=t)
    fam = "stream" if stream else "tile"
    assert f"family={fam} " in q.qdg_moe_describe(q.qdg_plan_create(layer, q.moe(top_k), tun), t, bm)
    y = _moe_gemm(layer, pk, H.bf16_dev(x), ids, bm, 0, top_k, tuning=tun)
    y64 = ref.moe_gemm_rows(x, ids, lambda e: ref.dequant_int4_sym(qs[e], ss[e]), input_is_per_pair=False)
    assert metrics.rel_frob(H.to_f64(y), y64) <= 2e-3
    # down projection: one input row per pair
    qd, sd = _experts(E, hid, inter, salt=2)
    layer_d, pk_d = _moe_packed(qd, sd, hid, inter)
    h = synth.moe_hidden_bf16_bits(t * top_k, inter, salt=t)
    yd = _moe_gemm(layer_d, pk_d, H.bf16_dev(h), ids, bm, 1, top_k, tuning=tun)
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
    # (16-row blocks of this short K default to the LDS-tiled family: the
    # streaming one is pinned by a tuning)
    tm = q.TuningConfig(block_n=64, waves=8 if pin_ws else 4) if bm == 16 else None
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
    # 16-row blocks: 16 x 512 tiles when K holds at most 16 groups
    assert fam == ("tile" if bm in (32, 64, 128) or k <= 2048 else "stream")
    xf = codecs.bf16_bits_to_f64(x)
    for p in pairs:
        e = int(ids.reshape(-1)[p])
        qv, s = quant.quantize_int4_sym(w_host[e])
        yr = xf[p if per_pair else p // top_k] @ ref.dequant_int4_sym(qv, s).T
        err = metrics.rel_frob(H.to_f64(y[p]), yr)
        print(f"MoE {proj} T={t} bm={bm} pair {p} expert {e}: rel_frob={err:.3e}")
        assert err <= 2e-3, (p, err)
        H.assert_elementwise(y[p], yr)
    # every real pair row was written (the output was prefilled with NaN)
    assert not torch.isnan(y.float()).any()


@pytest.mark.parametrize("t,bm,inter,stream", [(8, 16, 256, True), (64, 16, 144, True), (64, 16, 144, False),
                                                (64, 32, 256, False), (64, 32, 144, False), (300, 64, 256, False),
                                                (300, 64, 144, False), (300, 128, 256, False), (1024, 128, 144, False)])
@pytest.mark.parametrize("otype", [q.QDG_O_F32, q.QDG_O_BF16])
def test_moe_gate_up_silu_mul_epilogue(qdg, t, bm, inter, stream, otype):
    # fused gate+up (n = 2I) with the SiLU*mul epilogue: Y = silu(G) * U,
    # [T*top_k][I]; 16-row blocks pinned to the streaming family run four
    # tiles (two gate + two up) per workgroup, every other case here the
    # LDS-tiled family (I = 144: an odd number of gate tiles, so a
    # workgroup's tile slots run partly past the layer)
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
    tun = q.TuningConfig(block_n=64, waves=4) if stream else None
    plan = q.qdg_plan_create(layer, q.moe(top_k, epilogue=q.QDG_EPI_SILU_MUL), tun)
    desc = q.qdg_moe_describe(plan, t, bm)
    assert "epilogue=silu_mul" in desc and ("family=tile" in desc) == (not stream)
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


@pytest.mark.parametrize("t", [8, 64, 300])
@pytest.mark.parametrize("silu", [False, True])
def test_moe_16_row_tiles(qdg, t, silu):
    # a tuning with block_n 512 runs 16-row blocks as 16 x 512 tiles of the
    # LDS-tiled family (gate+up over token rows, with or without SiLU*mul;
    # down over pair rows); I = 144 leaves part of a workgroup's tile slots
    # past the layer
    E, top_k, hid, inter = 16, 4, 1024, 144
    tun = q.TuningConfig(block_m=16, block_n=512, waves=8)
    ids, _ = ref.route_topk(synth.router_logits(t, E, salt=t + 21), top_k)
    qs, ss = _experts(E, 2 * inter, hid, salt=13)
    x = synth.activations_bf16_bits(t, hid, workload_id=4, salt=t + 22)
    gu64 = ref.moe_gemm_rows(x, ids, lambda e: ref.dequant_int4_sym(qs[e], ss[e]), input_is_per_pair=False)
    layer, pk = _moe_packed(qs, ss, 2 * inter, hid)
    sid, blk, npad, cap = _align_dev(ids, E, 16)
    plan = q.qdg_plan_create(layer, q.moe(top_k, epilogue=q.QDG_EPI_SILU_MUL if silu else 0), tun)
    assert "family=tile block_m=16 block_n=512" in q.qdg_moe_describe(plan, t, 16)
    ws, nbytes = H.workspace(plan, t)
    y = H.out_tensor(t * top_k, inter if silu else 2 * inter, q.QDG_O_BF16)
    q.qdg_moe_gemm(plan, H.bf16_dev(x).data_ptr(), None, pk.buf.data_ptr(), sid.data_ptr(), blk.data_ptr(),
                   npad.data_ptr(), t, 16, 0, y.data_ptr(), ws.data_ptr(), nbytes, q.current_stream())
    torch.cuda.synchronize()
    assert not torch.isnan(y.float()).any()
    want = ref.silu_mul(gu64) if silu else gu64
    err = metrics.rel_frob(H.to_f64(y), want)
    print(f"16-row tiles T={t} silu={silu}: rel_frob={err:.3e}")
    assert err <= 2e-3, err
    if not silu:  # down projection (K = 256: whole groups of 128)
        qd, sd = _experts(E, hid, 256, salt=14)
        layer_d, pk_d = _moe_packed(qd, sd, hid, 256)
        h = synth.moe_hidden_bf16_bits(t * top_k, 256, salt=t + 23)
        yd = _moe_gemm(layer_d, pk_d, H.bf16_dev(h), ids, 16, 1, top_k, tuning=tun)
        yd64 = ref.moe_gemm_rows(h, ids, lambda e: ref.dequant_int4_sym(qd[e], sd[e]), input_is_per_pair=True)
        assert not torch.isnan(yd.float()).any()
        assert metrics.rel_frob(H.to_f64(yd), yd64) <= 2e-3


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


@pytest.mark.parametrize("t", [64, 1000])
def test_moe_combine_bf16_rows(qdg, t):
    # bf16 pair rows: the same fp32 chain as the f32 combine on the widened
    # rows (bit for bit), within 1e-6 / 2e-3 of the fp64 combine of the same
    # rows, and within 2e-3 of the combine of the unrounded rows with f32
    # output (the one bf16 rounding of the rows costs about 1.6e-3)
    top_k, n = 8, 7168
    r = np.random.default_rng(90 + t)
    y64 = r.normal(size=(t * top_k, n))
    yb = codecs.f32_to_bf16_bits(y64.astype(np.float32))
    w = r.uniform(0.0, 0.5, t * top_k).astype(np.float32)
    yb_dev, w_dev = H.bf16_dev(yb), H.dev(w)
    yw_dev = H.dev(codecs.bf16_bits_to_f64(yb).astype(np.float32))
    ref_same = ref.moe_combine(codecs.bf16_bits_to_f64(yb), w, top_k)
    for otype in (q.QDG_O_F32, q.QDG_O_BF16):
        out = H.out_tensor(t, n, otype)
        q.qdg_moe_combine_bf16(yb_dev.data_ptr(), w_dev.data_ptr(), t, top_k, n, out.data_ptr(), otype,
                               q.current_stream())
        out32 = H.out_tensor(t, n, otype)
        q.qdg_moe_combine(yw_dev.data_ptr(), w_dev.data_ptr(), t, top_k, n, out32.data_ptr(), otype,
                          q.current_stream())
        torch.cuda.synchronize()
        assert torch.equal(out, out32)
        err = metrics.rel_frob(H.to_f64(out), ref_same)
        assert err <= (1e-6 if otype == q.QDG_O_F32 else 2e-3), err
        if otype == q.QDG_O_F32:
            e2e = metrics.rel_frob(H.to_f64(out), ref.moe_combine(y64, w, top_k))
            print(f"combine of bf16 rows T={t}: {e2e:.3e} against the unrounded rows")
            assert e2e <= 2e-3, e2e


@pytest.mark.parametrize("bm", [16, 64])
def test_moe_empty_batch(qdg, bm):
    # T = 0: the sort yields no blocks (num_padded 0, every block entry -1,
    # every slot the sentinel T*top_k = 0) and the grouped GEMM and the
    # combine enqueue nothing (their outputs stay untouched)
    E, top_k, hid, n = 16, 4, 1024, 512
    sid, blk, npad, cap = _align_dev(np.zeros((0, top_k), np.int32), E, bm)
    assert int(npad.item()) == 0
    assert cap == q.qdg_moe_align_capacity(0, top_k, E, bm)
    assert torch.all(blk == -1) and torch.all(sid == 0)
    qs, ss = _experts(E, n, hid, salt=31)
    layer, pk = _moe_packed(qs, ss, n, hid)
    plan = q.qdg_plan_create(layer, q.moe(top_k))
    ws, nbytes = H.workspace(plan, 0)
    y = torch.full((4, n), 7.0, dtype=torch.bfloat16, device="cuda")
    dummy = torch.zeros(8, dtype=torch.int16, device="cuda")
    q.qdg_moe_gemm(plan, dummy.data_ptr(), None, pk.buf.data_ptr(), sid.data_ptr(), blk.data_ptr(),
                   npad.data_ptr(), 0, bm, 0, y.data_ptr(), ws.data_ptr(), nbytes, q.current_stream())
    w = torch.ones(4, dtype=torch.float32, device="cuda")
    yf = torch.zeros((4, n), dtype=torch.float32, device="cuda")
    q.qdg_moe_combine(yf.data_ptr(), w.data_ptr(), 0, top_k, n, y.data_ptr(), q.QDG_O_BF16, q.current_stream())
    torch.cuda.synchronize()
    assert torch.all(y.float() == 7.0)
