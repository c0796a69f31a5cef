"""Run-time compilation (qdg_plan_jit): the streaming-family instance that
hipRTC builds from the embedded source reproduces the ahead-of-time
instance's output bit for bit (the same source, target and options), and
both match the oracle; a second process loads the code object from the cache
directory instead of compiling it."""

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
        plan = q.qdg_plan_create(layer, q.moe(top_k))
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
