"""The allocation-free entry point (qdg_gemm_noalloc) against qdg_gemm with a
caller workspace: the same kernel instances on the same inputs, so every
output must match bit for bit. Two calls in a row, the second with a smaller
input (the scratch array keeps the first call's contents). The refusal of an
oversized request is host logic, tested on the CPU in test_abi."""

import numpy as np
import pytest
import torch

import quantized_dequant_gemm_amd as q
import synth
from oracle import quant
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _layer(n, k, salt):
    w = synth.weights_f32(n, k, workload_id=1, salt=salt)
    qv, s = quant.quantize_int4_sym(w)
    layer = q.layer_w4a16(n, k)
    qw, sc, _ = H.std_w4(qv, s)
    return layer, H.Packed(layer, qw, sc)


def _both(layer, pk, m, k, salt):
    plan = q.qdg_plan_create(layer, q.dense())
    a = H.bf16_dev(synth.activations_bf16_bits(m, k, workload_id=1, salt=salt))
    ws, nbytes = H.workspace(plan, m)
    assert nbytes > 64 * 1024 or m <= 16  # the case really uses the workspace
    y_ref = H.out_tensor(m, layer.n, layer.otype)
    y_na = H.out_tensor(m, layer.n, layer.otype)
    stream = q.current_stream()
    q.qdg_gemm(plan, a.data_ptr(), None, pk.buf.data_ptr(), y_ref.data_ptr(), m, ws.data_ptr(), nbytes, stream)
    q.qdg_gemm_noalloc(plan, a.data_ptr(), None, pk.buf.data_ptr(), y_na.data_ptr(), m, stream)
    torch.cuda.synchronize()
    return q.qdg_plan_describe(plan, m), y_ref, y_na


def test_noalloc_matches_workspace_entry_point(qdg):
    # first: the LDS-tiled family with a K split (fp32 partials and row sums
    # in the scratch array); second, smaller: weight streaming with a K split
    layer, pk = _layer(4096, 4096, salt=1)
    for m, fam in ((200, "tile"), (16, "wstream")):
        desc, y_ref, y_na = _both(layer, pk, m, 4096, salt=m)
        assert f"family={fam}" in desc and "split_k=1 " not in desc, desc
        assert not torch.isnan(y_ref.float()).any()
        assert torch.equal(y_na, y_ref), desc
