"""Grouped MoE with int8 / fp8 activations (W8A8, W4A8-INT8, W4A8-MXFP4)
against the oracle: every (token, slot) pair row equals its expert's dense
reference on that pair's input row (exact int32 accumulators with raw output,
relative Frobenius <= 1e-3 with fp32 and <= 2e-3 with bf16 output), every real
pair row is written and padding rows are never touched. 16- and 32-row
expert blocks run the streaming family, 64- and 128-row blocks the 8-bit
LDS-tiled one (64 x 512 and 128 x 256 tiles), in the instance that skips
all-padding 32-row halves of blocks while experts average at most one block
of rows."""

import numpy as np
import pytest
import torch

import quantized_dequant_gemm_amd as q
import synth
from oracle import codecs, metrics, quant, ref
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

E, TOP_K = 16, 4


def _align_dev(ids, bm):
    t, top_k = ids.shape
    cap = q.qdg_moe_align_capacity(t, top_k, E, bm)
    sid = torch.empty(cap, dtype=torch.int32, device="cuda")
    blk = torch.empty(cap // bm, dtype=torch.int32, device="cuda")
    npad = torch.zeros(1, dtype=torch.int32, device="cuda")
    q.qdg_moe_align(H.dev(ids.astype(np.int32)).data_ptr(), t, top_k, E, bm, sid.data_ptr(), blk.data_ptr(),
                    npad.data_ptr(), q.current_stream())
    torch.cuda.synchronize()
    return sid, blk, npad


def _experts(kind, n, k, salt):
    """Per-expert standard-format weights (stacked on device) and the oracle's
    dense reference of one expert on given activation rows."""
    ws = [synth.weights_f32(n, k, workload_id=5, salt=1000 * salt + e) for e in range(E)]
    if kind == "w8a8":
        qs = [quant.quantize_int8_per_channel(w) for w in ws]
        std = (H.dev(np.stack([x.astype(np.int8) for x, _ in qs])), H.dev(np.stack([s for _, s in qs])))
        return std, lambda e, qa, sa: ref.gemm_w8a8(qa, sa, qs[e][0], qs[e][1])
    if kind == "w4a8":
        qs = [quant.quantize_int4_sym(w) for w in ws]
        std = (H.dev(np.stack([codecs.pack_nibbles(codecs.encode_int4(v)) for v, _ in qs])),
               H.dev(np.stack([np.asarray(s, np.uint16).view(np.int16) for _, s in qs])))
        return std, lambda e, qa, sa: ref.gemm_w4a8(qa, sa, qs[e][0], qs[e][1])
    qs = [quant.quantize_mxfp4(w) for w in ws]
    std = (H.dev(np.stack([codecs.pack_nibbles(c) for c, _ in qs])), H.dev(np.stack([x for _, x in qs])))
    return std, lambda e, ac, sa: ref.gemm_mxfp4(ac, sa, qs[e][0], qs[e][1])


def _layer(kind, n, k, otype):
    mk = {"w8a8": q.layer_w8a8, "w4a8": q.layer_w4a8, "mxfp4": q.layer_mxfp4}[kind]
    return mk(n, k, otype=otype, num_experts=E)


def _acts(kind, rows, k, salt):
    a = synth.activations_bf16_bits(rows, k, workload_id=5, salt=salt)
    return quant.quantize_act_fp8(a) if kind == "mxfp4" else quant.quantize_act_int8(a)


@pytest.mark.parametrize("kind", ["w8a8", "w4a8", "mxfp4"])
@pytest.mark.parametrize("t,bm", [(8, 16), (64, 32), (200, 64), (300, 64), (1024, 64), (300, 128), (1024, 128)])
@pytest.mark.parametrize("per_pair", [0, 1])
def test_moe_8bit(qdg, kind, t, bm, per_pair):
    # gate+up reads token rows (per_pair 0), down one row per pair (1)
    n, k = (512, 1024) if not per_pair else (1024, 256)
    ids, _ = ref.route_topk(synth.router_logits(t, E, salt=t + 7 * per_pair), TOP_K)
    std, dense_ref = _experts(kind, n, k, salt=t + per_pair)
    rows_in = t * TOP_K if per_pair else t
    ac, sa = _acts(kind, rows_in, k, salt=3 * t + per_pair)
    y64, p = ref.moe_rows(ids, per_pair, lambda e, rows: dense_ref(e, ac[rows], sa[rows]))
    sid, blk, npad = _align_dev(ids, bm)
    a_dev, sa_dev = H.dev(ac), H.dev(sa)  # kept alive across the launches
    otypes = (q.QDG_O_F32, q.QDG_O_BF16) if kind == "mxfp4" else (q.QDG_O_I32, q.QDG_O_F32, q.QDG_O_BF16)
    for otype in otypes:
        layer = _layer(kind, n, k, otype)
        pk = H.Packed(layer, *std)
        plan = q.qdg_plan_create(layer, q.moe(TOP_K))
        d = q.qdg_moe_describe(plan, t, bm)
        assert ("family=qtile " if bm in (64, 128) else "family=stream ") in d, d
        # at most one block of rows per expert on average: the instance that
        # skips all-padding 32-row halves of blocks
        assert ("pad_skip=1" in d) == (bm in (64, 128) and t * TOP_K <= E * bm), d
        ws, nbytes = H.workspace(plan, t)
        y = H.out_tensor(t * TOP_K, n, otype)  # NaN / INT_MIN canary
        q.qdg_moe_gemm(plan, a_dev.data_ptr(), sa_dev.data_ptr(), pk.buf.data_ptr(), sid.data_ptr(),
                       blk.data_ptr(), npad.data_ptr(), t, bm, per_pair, y.data_ptr(), ws.data_ptr(), nbytes,
                       q.current_stream())
        torch.cuda.synchronize()
        if otype == q.QDG_O_I32:
            got = y.cpu().numpy().astype(np.int64)
            assert np.array_equal(got, p), f"{kind} raw accumulators differ"
        else:
            assert not torch.isnan(y.float()).any(), "a pair row was not written"
            err = metrics.rel_frob(H.to_f64(y), y64)
            print(f"{kind} T={t} bm={bm} per_pair={per_pair} otype={otype}: rel_frob={err:.3e}")
            assert err <= (1e-3 if otype == q.QDG_O_F32 else 2e-3), err


def test_moe_8bit_rejects_128_row_blocks_with_epilogue(qdg):
    layer = _layer("w4a8", 256, 256, q.QDG_O_BF16)
    plan = q.qdg_plan_create(layer, q.moe(TOP_K, epilogue=q.QDG_EPI_SILU_MUL))
    ws, nbytes = H.workspace(plan, 8)
    dummy = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    with pytest.raises(q.QdgError) as ex:
        q.qdg_moe_gemm(plan, dummy.data_ptr(), dummy.data_ptr(), dummy.data_ptr(), dummy.data_ptr(),
                       dummy.data_ptr(), dummy.data_ptr(), 8, 128, 0, dummy.data_ptr(), ws.data_ptr(), nbytes,
                       q.current_stream())
    assert ex.value.status == q.QDG_ERR_UNSUPPORTED


@pytest.mark.parametrize("kind", ["w4a8", "mxfp4"])
def test_moe_8bit_silu_mul_epilogue(qdg, kind):
    t, bm, n, k = 64, 16, 512, 1024
    ids, _ = ref.route_topk(synth.router_logits(t, E, salt=41), TOP_K)
    std, dense_ref = _experts(kind, n, k, salt=42)
    ac, sa = _acts(kind, t, k, salt=43)
    y64, _ = ref.moe_rows(ids, 0, lambda e, rows: dense_ref(e, ac[rows], sa[rows]))
    h64 = ref.silu_mul(y64)
    sid, blk, npad = _align_dev(ids, bm)
    a_dev, sa_dev = H.dev(ac), H.dev(sa)
    layer = _layer(kind, n, k, q.QDG_O_BF16)
    pk = H.Packed(layer, *std)
    plan = q.qdg_plan_create(layer, q.moe(TOP_K, epilogue=q.QDG_EPI_SILU_MUL))
    ws, nbytes = H.workspace(plan, t)
    y = H.out_tensor(t * TOP_K, n // 2, q.QDG_O_BF16)
    q.qdg_moe_gemm(plan, a_dev.data_ptr(), sa_dev.data_ptr(), pk.buf.data_ptr(), sid.data_ptr(), blk.data_ptr(),
                   npad.data_ptr(), t, bm, 0, y.data_ptr(), ws.data_ptr(), nbytes, q.current_stream())
    torch.cuda.synchronize()
    assert not torch.isnan(y.float()).any()
    err = metrics.rel_frob(H.to_f64(y), h64)
    assert err <= 2e-3, err
