"""Per-M-range autotuning against the oracle: after qdg_plan_autotune the
plan serves M's range with the fastest instance it timed, every result it
then produces matches the fp64 oracle to the format's tolerance (relative
Frobenius 2e-3 with bf16 output, 1e-3 with fp32 output of the 8-bit paths,
bit-exact raw int32), a new plan that takes the chosen tuning as its user
tuning reproduces the autotuned plan's output bit for bit, and the other M
ranges keep the heuristics."""

import numpy as np
import pytest
import torch

import quantized_dequant_gemm_amd as q
import synth
from oracle import metrics, quant, ref
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _run(plan, a_ptr, sa_ptr, pk, m, n, otype):
    ws, nbytes = H.workspace(plan, m)
    y = H.out_tensor(m, n, otype)
    q.qdg_gemm(plan, a_ptr, sa_ptr, pk.buf.data_ptr(), y.data_ptr(), m, ws.data_ptr(), nbytes, q.current_stream())
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("m", [1, 16, 40, 200])
def test_autotune_w4a16(qdg, m):
    n, k = 1024, 2048
    w = synth.weights_f32(n, k, workload_id=7, salt=m)
    qv, s = quant.quantize_int4_sym(w)
    a = synth.activations_bf16_bits(m, k, workload_id=7, salt=m)
    y64 = ref.gemm_w4a16(a, ref.dequant_int4_sym(qv, s))
    layer = q.layer_w4a16(n, k)
    pk = H.Packed(layer, *H.std_w4(qv, s)[:2])
    a_dev = H.bf16_dev(a)
    plan = q.qdg_plan_create(layer, q.dense())
    # a workspace for every candidate (split partials included)
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    y = H.out_tensor(m, n, layer.otype)
    chosen, us = q.qdg_plan_autotune(plan, a_dev.data_ptr(), None, pk.buf.data_ptr(), y.data_ptr(), m,
                                     ws.data_ptr(), ws.numel(), 5, q.current_stream())
    torch.cuda.synchronize()
    assert us > 0.0
    desc = q.qdg_plan_describe(plan, m)
    print(f"M={m}: {us:.2f} us  {desc.split(': ')[1]}")
    assert "tuning=autotuned" in desc
    assert metrics.rel_frob(H.to_f64(y), y64) <= 2e-3  # Y from the autotuning call
    # the same range (M in (2^(b-1), 2^b]) is served by the same instance; others are not
    lo = 1 if m == 1 else (1 << (int(m - 1).bit_length() - 1)) + 1
    assert "tuning=autotuned" in q.qdg_plan_describe(plan, lo)
    assert "tuning=heuristic" in q.qdg_plan_describe(plan, 4 * m + 64)
    ya = _run(plan, a_dev.data_ptr(), None, pk, m, n, layer.otype)
    assert metrics.rel_frob(H.to_f64(ya), y64) <= 2e-3
    # the chosen tuning as a user tuning: the same instance, bit for bit
    pu = q.qdg_plan_create(layer, q.dense(), chosen)
    assert q.qdg_plan_describe(pu, m).split("tuning=")[0] == desc.split("tuning=")[0]
    yu = _run(pu, a_dev.data_ptr(), None, pk, m, n, layer.otype)
    assert torch.equal(ya, yu)
    q.qdg_plan_autotune_reset(plan)
    assert "tuning=heuristic" in q.qdg_plan_describe(plan, m)


@pytest.mark.parametrize("otype", [q.QDG_O_I32, q.QDG_O_F32])
@pytest.mark.parametrize("m", [16, 100])
def test_autotune_w8a8(qdg, m, otype):
    n, k = 768, 1024
    w = synth.weights_f32(n, k, workload_id=7, salt=100 + m)
    qw, sw = quant.quantize_int8_per_channel(w)
    a = synth.activations_bf16_bits(m, k, workload_id=7, salt=100 + m)
    qa, sa = quant.quantize_act_int8(a)
    layer = q.layer_w8a8(n, k, otype=otype)
    pk = H.Packed(layer, H.dev(qw.astype(np.int8)), H.dev(sw))
    qa_dev, sa_dev = H.dev(qa), H.dev(sa)
    plan = q.qdg_plan_create(layer, q.dense())
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    y = H.out_tensor(m, n, otype)
    chosen, us = q.qdg_plan_autotune(plan, qa_dev.data_ptr(), sa_dev.data_ptr(), pk.buf.data_ptr(), y.data_ptr(), m,
                                     ws.data_ptr(), ws.numel(), 5, q.current_stream())
    torch.cuda.synchronize()
    print(f"M={m}: {us:.2f} us  {q.qdg_plan_describe(plan, m).split(': ')[1]}")
    assert "tuning=autotuned" in q.qdg_plan_describe(plan, m)
    ya = _run(plan, qa_dev.data_ptr(), sa_dev.data_ptr(), pk, m, n, otype)
    y64, acc = ref.gemm_w8a8(qa, sa, qw, sw)
    if otype == q.QDG_O_I32:
        assert np.array_equal(ya.cpu().numpy().astype(np.int64), acc)
        assert np.array_equal(y.cpu().numpy().astype(np.int64), acc)
    else:
        assert metrics.rel_frob(H.to_f64(ya), y64) <= 1e-3
        assert metrics.rel_frob(H.to_f64(y), y64) <= 1e-3
    pu = q.qdg_plan_create(layer, q.dense(), chosen)
    yu = _run(pu, qa_dev.data_ptr(), sa_dev.data_ptr(), pk, m, n, otype)
    assert torch.equal(ya, yu)


def test_autotune_respects_the_workspace(qdg):
    # with the heuristic instance's workspace only, every chosen instance fits it
    m, n, k = 16, 512, 4096
    w = synth.weights_f32(n, k, workload_id=7, salt=5)
    qv, s = quant.quantize_int4_sym(w)
    a = synth.activations_bf16_bits(m, k, workload_id=7, salt=5)
    layer = q.layer_w4a16(n, k)
    pk = H.Packed(layer, *H.std_w4(qv, s)[:2])
    a_dev = H.bf16_dev(a)
    plan = q.qdg_plan_create(layer, q.dense())
    ws, nbytes = H.workspace(plan, m)
    y = H.out_tensor(m, n, layer.otype)
    q.qdg_plan_autotune(plan, a_dev.data_ptr(), None, pk.buf.data_ptr(), y.data_ptr(), m, ws.data_ptr(), nbytes, 3,
                        q.current_stream())
    torch.cuda.synchronize()
    assert q.qdg_plan_workspace(plan, m) <= nbytes
    y64 = ref.gemm_w4a16(a, ref.dequant_int4_sym(qv, s))
    assert metrics.rel_frob(H.to_f64(_run(plan, a_dev.data_ptr(), None, pk, m, n, layer.otype)), y64) <= 2e-3
