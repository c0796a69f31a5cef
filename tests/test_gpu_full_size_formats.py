"""The further formats (W8A16, W4A16-NVFP4, W2A16, W4A4-MXFP4, MXFP4 x INT8)
at the layer sizes and in the launch configuration the benchmark times
(heuristic plan, default tuning): the mid-size batch (M = 256 at K = 4096,
M = 512 at the MXFP4 shapes, K split across workgroups) against the oracle on
every output, and M = 4096 on 40 sampled rows (every column), with each
format's tolerance: relative Frobenius <= 5e-5 (bf16-activation formats,
fp32 output), <= 1e-3 (8-bit / 4-bit activations, fp32 output) and
<= 2e-3 with bf16 output. Every output element must be written."""

import functools

import numpy as np
import pytest
import torch

import quantized_dequant_gemm_amd as q
import synth
from oracle import codecs, metrics, quant, ref
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

BF16_ACT = ("w8a16", "nvfp4", "w2a16")


@functools.lru_cache(maxsize=1)
def _weights(fmt, n, k):
    """Oracle-quantized weights: device standard-format tensors and a function
    that gives the oracle's fp64 product for given activation rows."""
    w = synth.weights_f32(n, k, workload_id=11, salt=n + 7 * k)
    if fmt == "w8a16":
        qw, sw = quant.quantize_int8_per_channel(w)
        std = (H.dev(qw.astype(np.int8)), H.dev(sw))
        return std, lambda a: ref.gemm_w8a16(a, qw, sw)
    if fmt == "nvfp4":
        codes, sc, ts = quant.quantize_nvfp4(w)
        std = (H.dev(codecs.pack_nibbles(codes)), H.dev(sc), None, H.dev(np.atleast_1d(np.asarray(ts, np.float32))))
        return std, lambda a: ref.gemm_nvfp4a16(a, codes, sc, ts)
    if fmt == "w2a16":
        qv, s, z = quant.quantize_uint2_asym(w)
        w64 = ref.dequant_uint2_asym(qv, s, z)
        std = (H.dev(codecs.pack_crumbs(qv)), H.dev(np.asarray(s, np.uint16).view(np.int16)), H.dev(z))
        return std, lambda a: ref.gemm_w4a16(a, w64)
    wc, we = quant.quantize_mxfp4(w)
    std = (H.dev(codecs.pack_nibbles(wc)), H.dev(we))
    if fmt == "w4a4":
        return std, lambda acts: ref.gemm_w4a4(acts[0], acts[1], wc, we)
    return std, lambda acts: ref.gemm_mxfp4_int8(acts[0], acts[1], wc, we)


def _layer(fmt, n, k, otype):
    mk = {"w8a16": q.layer_w8a16, "nvfp4": q.layer_nvfp4, "w2a16": q.layer_w2a16, "w4a4": q.layer_w4a4,
          "mxfp4_int8": q.layer_mxfp4_int8}[fmt]
    return mk(n, k, otype=otype)


def _run(fmt, m, n, k, rows):
    """Run the heuristic plan on M rows; compare the given rows (None: all)."""
    std, oracle_rows = _weights(fmt, n, k)
    a = synth.activations_bf16_bits(m, k, workload_id=11, salt=m + n)
    sel = slice(None) if rows is None else rows
    if fmt in BF16_ACT:
        a_dev, sa_dev = H.bf16_dev(a), None
        y64 = oracle_rows(a[sel])
    elif fmt == "w4a4":
        ac, ae = quant.quantize_act_mxfp4(a)
        a_dev, sa_dev = H.dev(codecs.pack_nibbles(ac)), H.dev(ae)
        y64 = oracle_rows((ac[sel], ae[sel]))
    else:
        qa, sa = quant.quantize_act_int8(a)
        a_dev, sa_dev = H.dev(qa), H.dev(sa)
        y64 = oracle_rows((qa[sel], sa[sel]))
    rows_d = None if rows is None else torch.from_numpy(rows).cuda()
    for otype in (q.QDG_O_F32, q.QDG_O_BF16):
        layer = _layer(fmt, n, k, otype)
        zeros = std[2] if len(std) > 2 else None
        tscale = std[3] if len(std) > 3 else None
        pk = H.Packed(layer, std[0], std[1], zeros, tscale)
        y, plan = H.gemm(layer, pk, a_dev, m, a_scales=sa_dev)
        d = q.qdg_plan_describe(plan, m)
        assert ("family=tile " if fmt in BF16_ACT else "family=qtile ") in d, d
        assert not torch.isnan(y.float()).any(), "an output element was not written"
        ys = y if rows_d is None else y[rows_d]
        err = metrics.rel_frob(H.to_f64(ys), y64)
        tol = 2e-3 if otype == q.QDG_O_BF16 else (5e-5 if fmt in BF16_ACT else 1e-3)
        print(f"{fmt} M={m} K={k} N={n} otype={otype} ({d.split('split_k=')[1].split()[0]} splits): "
              f"rel_frob={err:.3e}")
        assert err <= tol, err
        H.assert_elementwise(ys, y64)


def _sampled(m, seed):
    return np.unique(np.concatenate([[0, m - 1], np.random.default_rng(seed).integers(0, m, 38)]))


@pytest.mark.parametrize("fmt", ["w8a16", "nvfp4", "w2a16"])
@pytest.mark.parametrize("n", [4096, 14336])
def test_bf16_activation_formats(qdg, fmt, n):
    _run(fmt, 256, n, 4096, None)
    _run(fmt, 4096, n, 4096, _sampled(4096, n))


@pytest.mark.parametrize("fmt", ["w4a4", "mxfp4_int8"])
@pytest.mark.parametrize("k,n", [(7168, 2048), (2048, 7168)])
def test_mxfp4_weight_formats(qdg, fmt, k, n):
    _run(fmt, 512, n, k, None)
    _run(fmt, 4096, n, k, _sampled(4096, k))
