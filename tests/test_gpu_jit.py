"""Run-time compilation (qdg_plan_jit): the instance of every kernel family
(streaming, weight streaming in its resident and chunked forms, LDS-tiled,
8-bit LDS-tiled, 8-bit weight streaming, grouped MoE tiles) that hipRTC
builds from the embedded source reproduces the ahead-of-time instance's
output bit for bit (the same source, target and options), and both match
the oracle; a second process loads the code object from the cache directory
instead of compiling it."""

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import quantized_dequant_gemm_amd as q
import synth
from oracle import codecs, metrics, quant, ref
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(plan, a_ptr, sa_ptr, pk, m, n, otype):
    ws, nbytes = H.workspace(plan, m)
    y = H.out_tensor(m, n, otype)
    q.qdg_gemm(plan, a_ptr, sa_ptr, pk.buf.data_ptr(), y.data_ptr(), m, ws.data_ptr(), nbytes, q.current_stream())
    torch.cuda.synchronize()
    return y


def test_jit_w4a16_matches_aot_and_oracle(qdg, tmp_path):
    m, n, k = 24, 700, 2048
    w = synth.weights_f32(n, k, workload_id=10, salt=1)
    qv, s = quant.quantize_int4_sym(w)
    a = synth.activations_bf16_bits(m, k, workload_id=10, salt=2)
    layer = q.layer_w4a16(n, k)
    pk = H.Packed(layer, *H.std_w4(qv, s)[:2])
    a_dev = H.bf16_dev(a)
    aot = q.qdg_plan_create(layer, q.dense())
    jit = q.qdg_plan_create(layer, q.dense())
    info = q.qdg_plan_jit(jit, m, 0, str(tmp_path))
    print(f"compile {info.compile_ms:.0f} ms, load {info.load_ms:.1f} ms, {info.code_bytes} bytes, key {info.key.decode()}")
    assert info.from_cache in (0, 2) and info.code_bytes >= 0
    assert "code=jit" in q.qdg_plan_describe(jit, m) and "code=aot" in q.qdg_plan_describe(aot, m)
    y_aot = _run(aot, a_dev.data_ptr(), None, pk, m, n, layer.otype)
    y_jit = _run(jit, a_dev.data_ptr(), None, pk, m, n, layer.otype)
    assert torch.equal(y_aot, y_jit)
    assert metrics.rel_frob(H.to_f64(y_jit), ref.gemm_w4a16(a, ref.dequant_int4_sym(qv, s))) <= 2e-3
    # the same instance again in this process: no new compile
    again = q.qdg_plan_jit(q.qdg_plan_create(layer, q.dense()), m, 0, str(tmp_path))
    assert again.from_cache == 2 and again.compile_ms == 0.0
    if info.from_cache == 0:
        # a new process reads the code object from the cache directory
        code = ("import sys; sys.path.insert(0, %r); import quantized_dequant_gemm_amd as q; "
                "p = q.qdg_plan_create(q.layer_w4a16(%d, %d), q.dense()); i = q.qdg_plan_jit(p, %d, 0, %r); "
                "print(i.from_cache, i.compile_ms)") % (ROOT, n, k, m, str(tmp_path))
        out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
        assert out.returncode == 0, out.stderr[-2000:]
        fc, cms = out.stdout.split()[-2:]
        assert int(fc) == 1 and float(cms) == 0.0


@pytest.mark.parametrize("otype", [q.QDG_O_I32, q.QDG_O_F32])
def test_jit_w8a8_matches_aot(qdg, otype):
    m, n, k = 40, 300, 1024
    w = synth.weights_f32(n, k, workload_id=10, salt=3)
    qw, sw = quant.quantize_int8_per_channel(w)
    a = synth.activations_bf16_bits(m, k, workload_id=10, salt=4)
    qa, sa = quant.quantize_act_int8(a)
    layer = q.layer_w8a8(n, k, otype=otype)
    pk = H.Packed(layer, H.dev(qw.astype(np.int8)), H.dev(sw))
    qa_dev, sa_dev = H.dev(qa), H.dev(sa)
    aot = q.qdg_plan_create(layer, q.dense())
    jit = q.qdg_plan_create(layer, q.dense())
    q.qdg_plan_jit(jit, m)
    assert "family=stream" in q.qdg_plan_describe(jit, m) and "code=jit" in q.qdg_plan_describe(jit, m)
    y_aot = _run(aot, qa_dev.data_ptr(), sa_dev.data_ptr(), pk, m, n, otype)
    y_jit = _run(jit, qa_dev.data_ptr(), sa_dev.data_ptr(), pk, m, n, otype)
    assert torch.equal(y_aot, y_jit)
    y64, acc = ref.gemm_w8a8(qa, sa, qw, sw)
    if otype == q.QDG_O_I32:
        assert np.array_equal(y_jit.cpu().numpy().astype(np.int64), acc)
    else:
        assert metrics.rel_frob(H.to_f64(y_jit), y64) <= 1e-3


def test_jit_moe_matches_aot(qdg):
    E, top_k, t, bm = 4, 2, 48, 16
    n, k = 128, 512
    ids, _ = ref.route_topk(synth.router_logits(t, E, salt=9), top_k)
    qs = [quant.quantize_int4_sym(synth.weights_f32(n, k, workload_id=10, salt=50 + e)) for e in range(E)]
    layer = q.layer_w4a16(n, k, num_experts=E)
    qw = H.dev(np.stack([codecs.pack_nibbles(codecs.encode_int4(v)) for v, _ in qs]))
    sc = H.dev(np.stack([np.asarray(s_, np.uint16).view(np.int16) for _, s_ in qs]))
    pk = H.Packed(layer, qw, sc)
    a = synth.activations_bf16_bits(t, k, workload_id=10, salt=10)
    cap = q.qdg_moe_align_capacity(t, top_k, E, bm)
    sid = torch.empty(cap, dtype=torch.int32, device="cuda")
    blk = torch.empty(cap // bm, dtype=torch.int32, device="cuda")
    npad = torch.zeros(1, dtype=torch.int32, device="cuda")
    ids_dev = H.dev(ids.astype(np.int32))
    q.qdg_moe_align(ids_dev.data_ptr(), t, top_k, E, bm, sid.data_ptr(), blk.data_ptr(), npad.data_ptr(),
                    q.current_stream())
    a_dev = H.bf16_dev(a)
    outs = []
    for use_jit in (False, True):
        # the streaming family, pinned by the tuning (16-row blocks of a K
        # this short default to the LDS-tiled 16 x 512 tiles)
        plan = q.qdg_plan_create(layer, q.moe(top_k), q.TuningConfig(block_n=64, waves=4))
        if use_jit:
            q.qdg_plan_jit(plan, t, bm)
            assert "code=jit" in q.qdg_moe_describe(plan, t, bm)
        wsb = q.qdg_plan_workspace(plan, t)
        ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
        y = H.out_tensor(t * top_k, n, q.QDG_O_BF16)
        q.qdg_moe_gemm(plan, a_dev.data_ptr(), None, pk.buf.data_ptr(), sid.data_ptr(), blk.data_ptr(),
                       npad.data_ptr(), t, bm, 0, y.data_ptr(), ws.data_ptr(), wsb, q.current_stream())
        torch.cuda.synchronize()
        outs.append(y)
    assert torch.equal(outs[0], outs[1])


def test_jit_nvfp4_matches_aot(qdg):
    # the NVFP4 policy (hardware E2M1 convert, E4M3 block scales) built by hipRTC
    m, n, k = 24, 300, 1024
    codes, sc, ts = quant.quantize_nvfp4(synth.weights_f32(n, k, workload_id=10, salt=5))
    a = synth.activations_bf16_bits(m, k, workload_id=10, salt=6)
    layer = q.layer_nvfp4(n, k, otype=q.QDG_O_F32)
    pk = H.Packed(layer, H.dev(codecs.pack_nibbles(codes)), H.dev(sc),
                  tensor_scale=H.dev(np.array([ts], np.float32)))
    a_dev = H.bf16_dev(a)
    aot = q.qdg_plan_create(layer, q.dense())
    jit = q.qdg_plan_create(layer, q.dense())
    q.qdg_plan_jit(jit, m)
    assert "family=stream" in q.qdg_plan_describe(jit, m) and "code=jit" in q.qdg_plan_describe(jit, m)
    y_aot = _run(aot, a_dev.data_ptr(), None, pk, m, n, layer.otype)
    y_jit = _run(jit, a_dev.data_ptr(), None, pk, m, n, layer.otype)
    assert torch.equal(y_aot, y_jit)
    assert metrics.rel_frob(H.to_f64(y_jit), ref.gemm_nvfp4a16(a, codes, sc, ts)) <= 5e-5


def _w4a16_case(m, n, k, salt):
    qv, sc = quant.quantize_int4_sym(synth.weights_f32(n, k, workload_id=10, salt=salt))
    a = synth.activations_bf16_bits(m, k, workload_id=10, salt=salt + 1)
    layer = q.layer_w4a16(n, k)
    pk = H.Packed(layer, *H.std_w4(qv, sc)[:2])
    return layer, pk, H.bf16_dev(a), None, ref.gemm_w4a16(a, ref.dequant_int4_sym(qv, sc))


def _w8a8_case(m, n, k, salt):
    qw, sw = quant.quantize_int8_per_channel(synth.weights_f32(n, k, workload_id=10, salt=salt))
    qa, sa = quant.quantize_act_int8(synth.activations_bf16_bits(m, k, workload_id=10, salt=salt + 1))
    layer = q.layer_w8a8(n, k)
    pk = H.Packed(layer, H.dev(qw.astype(np.int8)), H.dev(sw))
    return layer, pk, H.dev(qa), H.dev(sa), ref.gemm_w8a8(qa, sa, qw, sw)[0]


def _w4a8_case(m, n, k, salt):
    qv, s16 = quant.quantize_int4_sym(synth.weights_f32(n, k, workload_id=10, salt=salt))
    qa, sa = quant.quantize_act_int8(synth.activations_bf16_bits(m, k, workload_id=10, salt=salt + 1))
    layer = q.layer_w4a8(n, k)
    pk = H.Packed(layer, *H.std_w4(qv, s16)[:2])
    return layer, pk, H.dev(qa), H.dev(sa), ref.gemm_w4a8(qa, sa, qv, s16)[0]


def _w4a4_case(m, n, k, salt):
    codes, e = quant.quantize_mxfp4(synth.weights_f32(n, k, workload_id=10, salt=salt))
    ac, ae = quant.quantize_act_mxfp4(synth.activations_bf16_bits(m, k, workload_id=10, salt=salt + 1))
    layer = q.layer_w4a4(n, k)
    pk = H.Packed(layer, H.dev(codecs.pack_nibbles(codes)), H.dev(e))
    return layer, pk, H.dev(codecs.pack_nibbles(ac)), H.dev(ae), ref.gemm_w4a4(ac, ae, codes, e)


def _w8a16_case(m, n, k, salt):
    qw, sw = quant.quantize_int8_per_channel(synth.weights_f32(n, k, workload_id=10, salt=salt))
    a = synth.activations_bf16_bits(m, k, workload_id=10, salt=salt + 1)
    layer = q.layer_w8a16(n, k)
    pk = H.Packed(layer, H.dev(qw.astype(np.int8)), H.dev(sw))
    return layer, pk, H.bf16_dev(a), None, ref.gemm_w8a16(a, qw, sw)


def _nvfp4_case(m, n, k, salt):
    codes, sc, ts = quant.quantize_nvfp4(synth.weights_f32(n, k, workload_id=10, salt=salt))
    a = synth.activations_bf16_bits(m, k, workload_id=10, salt=salt + 1)
    layer = q.layer_nvfp4(n, k)
    pk = H.Packed(layer, H.dev(codecs.pack_nibbles(codes)), H.dev(sc), None,
                  H.dev(np.atleast_1d(np.asarray(ts, np.float32))))
    return layer, pk, H.bf16_dev(a), None, ref.gemm_nvfp4a16(a, codes, sc, ts)


def _w2a16_case(m, n, k, salt):
    qv, sc, z = quant.quantize_uint2_asym(synth.weights_f32(n, k, workload_id=10, salt=salt))
    a = synth.activations_bf16_bits(m, k, workload_id=10, salt=salt + 1)
    layer = q.layer_w2a16(n, k)
    pk = H.Packed(layer, H.dev(codecs.pack_crumbs(qv)), H.dev(np.asarray(sc, np.uint16).view(np.int16)), H.dev(z))
    return layer, pk, H.bf16_dev(a), None, ref.gemm_w4a16(a, ref.dequant_uint2_asym(qv, sc, z))


# (family in the plan's description, kernel, case builder, M, N, K, tuning)
FAMILIES = {
    "tile": ("tile", _w4a16_case, 200, 1000, 2048, None),
    "wstream": ("wstream", _w4a16_case, 16, 1000, 2048, None),
    "wstream_chunked": ("wstream", _w4a16_case, 4, 512, 8192, dict(block_m=16, block_n=64, split_k=1, waves=8)),
    "wstream_split": ("wstream", _w4a16_case, 16, 256, 4096, dict(block_m=16, block_n=64, split_k=4, waves=8)),
    "qtile_split": ("qtile", _w8a8_case, 256, 512, 1024, dict(block_m=128, split_k=2)),
    "wstream8": ("wstream", _w8a8_case, 16, 2048, 4096, None),
    "qtile_w4a8": ("qtile", _w4a8_case, 256, 512, 1024, dict(block_m=128)),
    "qtile_w4a4": ("qtile", _w4a4_case, 256, 512, 1024, dict(block_m=128)),
    "stream_w4a4": ("stream", _w4a4_case, 32, 512, 1024, None),
    "tile_w8a16": ("tile", _w8a16_case, 200, 600, 1024, None),
    "tile_nvfp4": ("tile", _nvfp4_case, 200, 600, 1024, None),
    "tile_w2a16": ("tile", _w2a16_case, 200, 600, 1024, None),
}


@pytest.mark.parametrize("case", list(FAMILIES))
def test_jit_every_family_matches_aot(qdg, tmp_path, case):
    fam, build, m, n, k, tun = FAMILIES[case]
    layer, pk, a_dev, sa_dev, y64 = build(m, n, k, salt=len(case))
    tuning = q.TuningConfig(**tun) if tun else None
    aot = q.qdg_plan_create(layer, q.dense(), tuning)
    jit = q.qdg_plan_create(layer, q.dense(), tuning)
    assert f"family={fam} " in q.qdg_plan_describe(aot, m)
    info = q.qdg_plan_jit(jit, m, 0, str(tmp_path))
    print(f"{case}: compile {info.compile_ms:.0f} ms, {info.code_bytes} bytes")
    assert info.code_bytes > 0 or info.from_cache == 2
    assert "code=jit" in q.qdg_plan_describe(jit, m) and "code=aot" in q.qdg_plan_describe(aot, m)
    sa_ptr = sa_dev.data_ptr() if sa_dev is not None else None
    y_aot = _run(aot, a_dev.data_ptr(), sa_ptr, pk, m, n, layer.otype)
    y_jit = _run(jit, a_dev.data_ptr(), sa_ptr, pk, m, n, layer.otype)
    assert torch.equal(y_aot, y_jit)
    err = metrics.rel_frob(H.to_f64(y_jit), y64)
    assert err <= 2e-3, err


def test_jit_moe_tile_matches_aot(qdg, tmp_path):
    # grouped MoE in 32-row expert blocks (LDS-tiled 32 x 512 tiles)
    E, top_k, t, n, k, bm = 4, 2, 100, 512, 1024, 32
    ids, _ = ref.route_topk(synth.router_logits(t, E, salt=61), top_k)
    qs = [quant.quantize_int4_sym(synth.weights_f32(n, k, workload_id=10, salt=300 + e)) for e in range(E)]
    a = synth.activations_bf16_bits(t, k, workload_id=10, salt=62)
    layer = q.layer_w4a16(n, k, num_experts=E)
    pk = H.Packed(layer, H.dev(np.stack([codecs.pack_nibbles(codecs.encode_int4(qv)) for qv, _ in qs])),
                  H.dev(np.stack([np.asarray(sc, np.uint16).view(np.int16) for _, sc in qs])))
    cap = q.qdg_moe_align_capacity(t, top_k, E, bm)
    sid = torch.empty(cap, dtype=torch.int32, device="cuda")
    blk = torch.empty(cap // bm, dtype=torch.int32, device="cuda")
    npad = torch.zeros(1, dtype=torch.int32, device="cuda")
    ids_dev = H.dev(ids.astype(np.int32))
    q.qdg_moe_align(ids_dev.data_ptr(), t, top_k, E, bm, sid.data_ptr(), blk.data_ptr(), npad.data_ptr(),
                    q.current_stream())
    a_dev = H.bf16_dev(a)
    outs = []
    for use_jit in (False, True):
        plan = q.qdg_plan_create(layer, q.moe(top_k))
        if use_jit:
            q.qdg_plan_jit(plan, t, bm, str(tmp_path))
        d = q.qdg_moe_describe(plan, t, bm)
        assert "family=tile " in d and ("code=jit" if use_jit else "code=aot") in d, d
        ws, nbytes = H.workspace(plan, t)
        y = H.out_tensor(t * top_k, n, layer.otype)
        q.qdg_moe_gemm(plan, a_dev.data_ptr(), None, pk.buf.data_ptr(), sid.data_ptr(), blk.data_ptr(),
                       npad.data_ptr(), t, bm, 0, y.data_ptr(), ws.data_ptr(), nbytes, q.current_stream())
        torch.cuda.synchronize()
        outs.append(y)
    assert torch.equal(outs[0], outs[1])
    y64, _ = ref.moe_rows(ids, 0, lambda e, rows: ref.gemm_w4a16(a[rows], ref.dequant_int4_sym(*qs[e])))
    assert metrics.rel_frob(H.to_f64(outs[1]), y64) <= 2e-3


@pytest.mark.parametrize("per_pair", [0, 1])
def test_jit_moe_qtile_matches_aot(qdg, tmp_path, per_pair):
    # grouped MoE with int8 activations in 64-row expert blocks (8-bit
    # LDS-tiled 64 x 512 tiles); per_pair 1 reads one input row per pair
    E, top_k, t, n, k, bm = 8, 2, 160, 512, 1024, 64
    ids, _ = ref.route_topk(synth.router_logits(t, E, salt=71 + per_pair), top_k)
    qs = [quant.quantize_int4_sym(synth.weights_f32(n, k, workload_id=10, salt=400 + e)) for e in range(E)]
    rows_in = t * top_k if per_pair else t
    qa, sa = quant.quantize_act_int8(synth.activations_bf16_bits(rows_in, k, workload_id=10, salt=72))
    layer = q.layer_w4a8(n, k, num_experts=E)
    pk = H.Packed(layer, H.dev(np.stack([codecs.pack_nibbles(codecs.encode_int4(qv)) for qv, _ in qs])),
                  H.dev(np.stack([np.asarray(sc, np.uint16).view(np.int16) for _, sc in qs])))
    cap = q.qdg_moe_align_capacity(t, top_k, E, bm)
    sid = torch.empty(cap, dtype=torch.int32, device="cuda")
    blk = torch.empty(cap // bm, dtype=torch.int32, device="cuda")
    npad = torch.zeros(1, dtype=torch.int32, device="cuda")
    ids_dev = H.dev(ids.astype(np.int32))
    q.qdg_moe_align(ids_dev.data_ptr(), t, top_k, E, bm, sid.data_ptr(), blk.data_ptr(), npad.data_ptr(),
                    q.current_stream())
    qa_dev, sa_dev = H.dev(qa), H.dev(sa)
    outs = []
    for use_jit in (False, True):
        plan = q.qdg_plan_create(layer, q.moe(top_k))
        if use_jit:
            q.qdg_plan_jit(plan, t, bm, str(tmp_path))
        d = q.qdg_moe_describe(plan, t, bm)
        assert "family=qtile " in d and ("code=jit" if use_jit else "code=aot") in d, d
        ws, nbytes = H.workspace(plan, t)
        y = H.out_tensor(t * top_k, n, layer.otype)
        q.qdg_moe_gemm(plan, qa_dev.data_ptr(), sa_dev.data_ptr(), pk.buf.data_ptr(), sid.data_ptr(),
                       blk.data_ptr(), npad.data_ptr(), t, bm, per_pair, y.data_ptr(), ws.data_ptr(), nbytes,
                       q.current_stream())
        torch.cuda.synchronize()
        outs.append(y)
    assert torch.equal(outs[0], outs[1])
    y64, _ = ref.moe_rows(ids, per_pair, lambda e, rows: ref.gemm_w4a8(qa[rows], sa[rows], *qs[e])[0])
    assert metrics.rel_frob(H.to_f64(outs[1]), y64) <= 2e-3


def test_jit_plan_through_noalloc_entry_point(qdg, tmp_path):
    # a run-time-compiled plan through the allocation-free entry point: the
    # same output as the workspace entry point, in the LDS-tiled family with
    # its K split (partials in the library's scratch array)
    layer, pk, a_dev, _, y64 = _w4a16_case(200, 4096, 4096, salt=91)
    plan = q.qdg_plan_create(layer, q.dense())
    q.qdg_plan_jit(plan, 200, 0, str(tmp_path))
    d = q.qdg_plan_describe(plan, 200)
    assert "family=tile " in d and "code=jit" in d and "split_k=1 " not in d, d
    y_ws = _run(plan, a_dev.data_ptr(), None, pk, 200, 4096, layer.otype)
    y_na = H.out_tensor(200, 4096, layer.otype)
    q.qdg_gemm_noalloc(plan, a_dev.data_ptr(), None, pk.buf.data_ptr(), y_na.data_ptr(), 200, q.current_stream())
    torch.cuda.synchronize()
    assert torch.equal(y_ws, y_na)
    assert metrics.rel_frob(H.to_f64(y_na), y64) <= 2e-3
