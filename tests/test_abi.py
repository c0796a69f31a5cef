"""The C ABI on the CPU: the library loads, exports every symbol include/qdg.h
declares, and its host-side validation rejects bad input with the documented
status before any device work (no compute call runs here)."""

import ctypes
import os
import re

import pytest

import quantized_dequant_gemm_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "qdg.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qdg_[a-z_0-9]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert _declared() == sorted(q.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(q.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_version_and_empty_error():
    assert "gfx950" in q.qdg_version()


def _status(fn, *a):
    try:
        fn(*a)
    except q.QdgError as e:
        return e.status
    return q.QDG_OK


def test_layer_validation_codes():
    assert _status(q.qdg_validate_layer, q.layer_w4a16(4096, 4096)) == q.QDG_OK
    assert _status(q.qdg_validate_layer, q.layer_w4a16(4096, 1000)) == q.QDG_ERR_UNSUPPORTED  # K % 128
    bad = q.layer_w4a16(0, 128)
    assert _status(q.qdg_validate_layer, bad) == q.QDG_ERR_INVALID_ARG
    l = q.layer_w4a16(64, 128)
    l.group_size = 64
    assert _status(q.qdg_validate_layer, l) == q.QDG_ERR_UNSUPPORTED
    l = q.layer_w4a16(64, 128)
    l.has_zeros = 1  # symmetric int4 with zeros is contradictory
    assert _status(q.qdg_validate_layer, l) == q.QDG_ERR_INVALID_ARG
    l = q.layer_w4a16(64, 128, otype=q.QDG_O_I32)
    assert _status(q.qdg_validate_layer, l) == q.QDG_ERR_UNSUPPORTED
    l = q.layer_mxfp4(64, 128)
    l.atype = q.QDG_A_INT8  # MXFP4 x int8 takes per-token scales (act_group 0), not groups of 128
    assert _status(q.qdg_validate_layer, l) == q.QDG_ERR_UNSUPPORTED
    l = q.layer_w4a16(64, 128)
    l.arch = 942
    assert _status(q.qdg_validate_layer, l) == q.QDG_ERR_UNSUPPORTED
    assert "gfx950" in q.qdg_last_error()


def test_plan_and_workspace_validation():
    l = q.layer_w4a16(4096, 14336)
    p = q.qdg_plan_create(l, q.dense())
    assert q.qdg_plan_workspace(p, 16) >= 64 * 1024
    assert "split_k=" in q.qdg_plan_describe(p, 16)
    assert _status(q.qdg_plan_create, l, q.dense(), q.TuningConfig(block_m=48)) == q.QDG_ERR_UNSUPPORTED
    # a grouped plan over a one-expert layer is valid (E = 1 is the dense special case)
    assert _status(q.qdg_plan_create, l, q.moe(8)) == q.QDG_OK
    lm = q.layer_w4a16(4096, 7168, num_experts=256)
    assert _status(q.qdg_plan_create, lm, q.dense()) == q.QDG_ERR_INVALID_ARG
    assert _status(q.qdg_plan_create, lm, q.moe(0)) == q.QDG_ERR_INVALID_ARG
    # grouped MoE: W4A16 with int4 symmetric weights and the int8 / fp8
    # activation formats (streaming family, 16- to 64-row blocks)
    la = q.layer_w4a16(4096, 7168, asym=True, num_experts=8)
    assert _status(q.qdg_plan_create, la, q.moe(8)) == q.QDG_ERR_UNSUPPORTED
    for mk in (q.layer_w8a8, q.layer_w4a8, q.layer_mxfp4):
        p8 = q.qdg_plan_create(mk(4096, 2048, num_experts=8), q.moe(8))
        assert "family=stream" in q.qdg_moe_describe(p8, 64, 32)
        # 128-row blocks: the 8-bit LDS-tiled family, without an epilogue
        assert "family=qtile" in q.qdg_moe_describe(p8, 4096, 128)
        p8s = q.qdg_plan_create(mk(4096, 2048, num_experts=8), q.moe(8, epilogue=q.QDG_EPI_SILU_MUL))
        with pytest.raises(q.QdgError):
            q.qdg_moe_describe(p8s, 64, 128)


def test_describe_reports_the_instance_that_runs():
    # dense W4A16: weight streaming at M = 16, 32 x 32 MFMA blocks in the tiled family at large M
    p = q.qdg_plan_create(q.layer_w4a16(14336, 4096), q.dense())
    assert "family=wstream" in q.qdg_plan_describe(p, 16)
    big = q.qdg_plan_describe(p, 8192)
    assert "family=tile" in big and "mfma=32x32x16_bf16" in big and "waves=8" in big
    p8 = q.qdg_plan_create(q.layer_w8a8(14336, 4096), q.dense())
    assert "mfma=16x16x64_i8" in q.qdg_plan_describe(p8, 4096)
    # mid M: one partly filled 128-row block of the tiled families
    assert "family=stream" in q.qdg_plan_describe(p, 32)
    assert "family=tile" in q.qdg_plan_describe(p, 33)
    assert "family=stream" in q.qdg_plan_describe(p8, 63)
    assert "family=qtile" in q.qdg_plan_describe(p8, 64)
    # ... but up to 128 rows the streaming family keeps fp4 x fp4 layers and
    # int8 x int8 layers whose streaming grid is small enough to be split
    narrow8 = q.qdg_plan_create(q.layer_w8a8(4096, 4096), q.dense())
    assert "family=stream" in q.qdg_plan_describe(narrow8, 128)
    assert "family=qtile" in q.qdg_plan_describe(narrow8, 129)
    w4a8 = q.qdg_plan_create(q.layer_w4a8(4096, 4096), q.dense())
    assert "family=qtile" in q.qdg_plan_describe(w4a8, 64)
    w4a4 = q.qdg_plan_create(q.layer_w4a4(2048, 7168), q.dense())
    assert "family=stream" in q.qdg_plan_describe(w4a4, 128)
    assert "family=qtile" in q.qdg_plan_describe(w4a4, 129)
    # batch-invariant plans never switch family with M
    pb = q.qdg_plan_create(q.layer_w4a16(14336, 4096), q.dense(batch_invariant=1))
    assert "family=stream" in q.qdg_plan_describe(pb, 100)
    # grouped MoE: the caller's block size picks the family
    pm = q.qdg_plan_create(q.layer_w4a16(4096, 7168, num_experts=256), q.moe(8))
    d16 = q.qdg_moe_describe(pm, 64, 16)
    assert "family=stream" in d16 and "block_n=64" in d16
    pw = q.qdg_plan_create(q.layer_w4a16(4096, 7168, num_experts=256), q.moe(8), q.TuningConfig(block_n=64, waves=8))
    assert "family=wstream" in q.qdg_moe_describe(pw, 64, 16)
    assert "family=tile" in q.qdg_moe_describe(pm, 512, 32) and "block_m=32 " in q.qdg_moe_describe(pm, 512, 32)
    pmb = q.qdg_plan_create(q.layer_w4a16(4096, 7168, num_experts=256), q.moe(8, batch_invariant=1))
    assert "family=stream" in q.qdg_moe_describe(pmb, 512, 32)
    assert "family=tile" in q.qdg_moe_describe(pm, 4096, 128)
    with pytest.raises(q.QdgError):
        q.qdg_moe_describe(pm, 64, 48)
    with pytest.raises(q.QdgError):
        q.qdg_moe_describe(p, 64, 16)  # not a MoE plan


def test_epilogue_and_combine_validation():
    lm = q.layer_w4a16(4096, 7168, num_experts=8)
    silu = q.QDG_EPI_SILU_MUL
    p = q.qdg_plan_create(lm, q.moe(8, epilogue=silu))
    assert "epilogue=silu_mul" in q.qdg_moe_describe(p, 64, 16)
    assert "family=stream" in q.qdg_moe_describe(p, 64, 16)  # weight streaming has no such epilogue
    assert _status(q.qdg_plan_create, q.layer_w4a16(4096, 7168), q.ComputeConfig(
        kind=q.QDG_KIND_DENSE, batch_invariant=0, top_k=0, epilogue=silu)) == q.QDG_ERR_UNSUPPORTED
    assert _status(q.qdg_plan_create, q.layer_w4a16(4112, 7168, num_experts=8),
                   q.moe(8, epilogue=silu)) == q.QDG_ERR_UNSUPPORTED  # I = 2056 is no multiple of 16
    assert _status(q.qdg_plan_create, q.layer_w4a8(4096, 7168, otype=q.QDG_O_I32, num_experts=8),
                   q.moe(8, epilogue=silu)) == q.QDG_ERR_UNSUPPORTED
    assert _status(q.qdg_plan_create, lm, q.moe(8, epilogue=7)) == q.QDG_ERR_INVALID_ARG
    # combine: argument checks before any device work
    assert _status(q.qdg_moe_combine, 1, 1, 4, 8, 64, 1, q.QDG_O_I32) == q.QDG_ERR_INVALID_ARG
    assert _status(q.qdg_moe_combine, 16, 16, 4, 8, 66, 16, q.QDG_O_BF16) == q.QDG_ERR_UNSUPPORTED
    assert _status(q.qdg_moe_combine, 16, 16, 4, 8, 64, 8, q.QDG_O_BF16) == q.QDG_ERR_MISALIGNED
    q.qdg_moe_combine(0, 0, 0, 8, 64, 0, q.QDG_O_BF16)  # T = 0 enqueues nothing
    assert _status(q.qdg_moe_combine_bf16, 1, 1, 4, 8, 64, 1, q.QDG_O_I32) == q.QDG_ERR_INVALID_ARG
    assert _status(q.qdg_moe_combine_bf16, 16, 16, 4, 8, 66, 16, q.QDG_O_BF16) == q.QDG_ERR_UNSUPPORTED
    assert _status(q.qdg_moe_combine_bf16, 8, 16, 4, 8, 64, 8, q.QDG_O_BF16) == q.QDG_ERR_MISALIGNED
    assert _status(q.qdg_moe_combine_bf16, 4, 16, 4, 8, 64, 16, q.QDG_O_BF16) == q.QDG_ERR_MISALIGNED
    q.qdg_moe_combine_bf16(0, 0, 0, 8, 64, 0, q.QDG_O_BF16)  # T = 0 enqueues nothing


def test_gemm_argument_errors_before_device_work():
    l = q.layer_w4a16(64, 128)
    p = q.qdg_plan_create(l, q.dense())
    ws = q.qdg_plan_workspace(p, 4)
    # NULL operands, misaligned A, short workspace: all rejected on the host
    assert _status(q.qdg_gemm, p, 0, None, 256, 256, 4, 256, ws, 0) == q.QDG_ERR_INVALID_ARG
    assert _status(q.qdg_gemm, p, 0x1008, None, 256, 256, 4, 256, ws, 0) == q.QDG_ERR_MISALIGNED
    assert _status(q.qdg_gemm, p, 0x1000, None, 256, 256, 4, 256, ws - 1, 0) == q.QDG_ERR_WORKSPACE
    assert _status(q.qdg_gemm, p, 0x1000, None, 256, 256, -1, 256, ws, 0) == q.QDG_ERR_INVALID_ARG
    assert _status(q.qdg_gemm, p, 0, None, 0, 0, 0, 0, 0, 0) == q.QDG_OK  # M = 0: nothing to do
    l8 = q.layer_w8a8(64, 128)
    p8 = q.qdg_plan_create(l8, q.dense())
    assert _status(q.qdg_gemm, p8, 0x1000, None, 256, 256, 4, 256, 1 << 20, 0) == q.QDG_ERR_INVALID_ARG


def test_preprocess_and_moe_validation():
    l = q.layer_w4a16(100, 256)
    n = q.qdg_preprocess_query(l)
    assert n % 256 == 0 and n >= 112 * 256 // 2
    w = q.StdWeights(qweight=0x1000, scales=0x2000, zeros=None)
    assert _status(q.qdg_preprocess, l, w, 0x10000, n - 1, 0) == q.QDG_ERR_INVALID_ARG
    assert _status(q.qdg_preprocess, l, w, 0x10010, n, 0) == q.QDG_ERR_MISALIGNED
    la = q.layer_w4a16(100, 256, asym=True)
    assert _status(q.qdg_preprocess, la, w, 0x10000, 1 << 20, 0) == q.QDG_ERR_INVALID_ARG  # zeros missing
    assert q.qdg_moe_align_capacity(64, 8, 256, 16) == 512 + 256 * 15
    assert _status(q.qdg_moe_align_capacity, 64, 8, 256, 24) == q.QDG_ERR_UNSUPPORTED
    assert _status(q.qdg_moe_align_capacity, 64, 8, 2048, 16) == q.QDG_ERR_UNSUPPORTED


def test_autotune_validation_before_device_work():
    l = q.layer_w4a16(64, 128)
    p = q.qdg_plan_create(l, q.dense())
    at = q.qdg_plan_autotune
    # MoE, user-tuned and batch-invariant plans are not autotuned
    pm = q.qdg_plan_create(q.layer_w4a16(64, 128, num_experts=2), q.moe(1))
    assert _status(at, pm, 0x1000, None, 256, 256, 4, 256, 1 << 20, 5, 0) == q.QDG_ERR_UNSUPPORTED
    pu = q.qdg_plan_create(l, q.dense(), q.TuningConfig(block_m=16))
    assert _status(at, pu, 0x1000, None, 256, 256, 4, 256, 1 << 20, 5, 0) == q.QDG_ERR_UNSUPPORTED
    pb = q.qdg_plan_create(l, q.dense(batch_invariant=1))
    assert _status(at, pb, 0x1000, None, 256, 256, 4, 256, 1 << 20, 5, 0) == q.QDG_ERR_UNSUPPORTED
    # bad M, reps and NULL operands
    assert _status(at, p, 0x1000, None, 256, 256, 0, 256, 1 << 20, 5, 0) == q.QDG_ERR_INVALID_ARG
    assert _status(at, p, 0x1000, None, 256, 256, 4, 256, 1 << 20, 0, 0) == q.QDG_ERR_INVALID_ARG
    assert _status(at, p, 0x1000, None, 256, 256, 4, 256, 1 << 20, 1001, 0) == q.QDG_ERR_INVALID_ARG
    assert _status(at, p, 0, None, 256, 256, 4, 256, 1 << 20, 5, 0) == q.QDG_ERR_INVALID_ARG
    assert _status(at, p, 0x1000, None, 256, 256, 4, 0, 1 << 20, 5, 0) == q.QDG_ERR_INVALID_ARG
    # nothing was recorded: the heuristics still serve every M
    q.qdg_plan_autotune_reset(p)
    assert all("tuning=heuristic" in q.qdg_plan_describe(p, m) for m in (1, 16, 100, 5000))


def test_w4a4_layer_validation():
    # MXFP4 weights take fp8 activations with 128-groups or MXFP4 activations with 32-blocks
    q.qdg_validate_layer(q.layer_w4a4(64, 256))  # raises on a bad layer
    bad = q.layer_w4a4(64, 256)
    bad.act_group = 128
    assert _status(q.qdg_plan_create, bad, q.dense()) == q.QDG_ERR_UNSUPPORTED
    p = q.qdg_plan_create(q.layer_w4a4(64, 256), q.dense())
    for m in (1, 16, 200, 5000):
        d = q.qdg_plan_describe(p, m)
        assert "w4a4-mxfp4" in d and ("family=stream" if m <= 128 else "family=qtile") in d and "f4f4" in d
    pm = q.qdg_plan_create(q.layer_w4a4(64, 256, num_experts=4), q.moe(2))
    assert "family=stream" in q.qdg_moe_describe(pm, 8, 16)
    # the scales are required
    assert _status(q.qdg_gemm, p, 0x1000, None, 256, 256, 4, 256, 1 << 20, 0) == q.QDG_ERR_INVALID_ARG


def test_w8a16_layer_validation():
    q.qdg_validate_layer(q.layer_w8a16(64, 256))
    p = q.qdg_plan_create(q.layer_w8a16(64, 256), q.dense())
    for m in (1, 16, 32, 33, 200):
        d = q.qdg_plan_describe(p, m)
        fam, mfma = ("family=stream", "16x16x32_bf16") if m <= 32 else ("family=tile", "32x32x16_bf16")
        assert "w8a16-int8" in d and fam in d and mfma in d, d
    bad = q.layer_w8a16(64, 256, otype=q.QDG_O_I32)
    assert _status(q.qdg_validate_layer, bad) == q.QDG_ERR_UNSUPPORTED


def test_jit_validation_before_device_work():
    p = q.qdg_plan_create(q.layer_w4a16(14336, 4096), q.dense())
    assert _status(q.qdg_plan_jit, p, 0) == q.QDG_ERR_INVALID_ARG
    # a MoE block size no family serves is rejected before any compile
    pm = q.qdg_plan_create(q.layer_w4a16(4096, 7168, num_experts=8), q.moe(8))
    assert _status(q.qdg_plan_jit, pm, 64, 48) == q.QDG_ERR_UNSUPPORTED
    for m in (1, 16, 24, 200, 5000):  # every family starts ahead of time
        assert "code=aot" in q.qdg_plan_describe(p, m)
    # the fp8 x fp4 scaled-MFMA formats are not compiled at run time
    for layer in (q.layer_mxfp4(2048, 7168), q.layer_mxfp4_int8(2048, 7168)):
        for m in (16, 32, 512):
            assert _status(q.qdg_plan_jit, q.qdg_plan_create(layer, q.dense()), m) == q.QDG_ERR_UNSUPPORTED


def test_nvfp4_layer_validation():
    # NVFP4 weights: E4M3 scales per 16, bf16 activations, no zeros, float output
    q.qdg_validate_layer(q.layer_nvfp4(64, 256))
    for field, value in (("group_size", 32), ("stype", q.QDG_S_E8M0), ("atype", q.QDG_A_INT8), ("has_zeros", 1),
                         ("otype", q.QDG_O_I32)):
        bad = q.layer_nvfp4(64, 256)
        setattr(bad, field, value)
        assert _status(q.qdg_validate_layer, bad) == q.QDG_ERR_UNSUPPORTED, field
    p = q.qdg_plan_create(q.layer_nvfp4(64, 256), q.dense())
    for m in (1, 16, 32, 33, 64, 200, 5000):
        d = q.qdg_plan_describe(p, m)
        fam, mfma = ("family=stream", "16x16x32_bf16") if m <= 32 else ("family=tile", "32x32x16_bf16")
        assert "w4a16-nvfp4" in d and fam in d and mfma in d, d
    # 16-row blocks of a layer with >= 256 tiles: one tile per workgroup, no K split
    d = q.qdg_plan_describe(q.qdg_plan_create(q.layer_nvfp4(4096, 4096), q.dense()), 16)
    assert "block_n=16" in d and "split_k=1" in d, d
    # the tiled NVFP4 instance is 128 x 256 with 8 waves only
    t4 = q.TuningConfig(block_m=128, waves=4)
    assert _status(q.qdg_plan_create, q.layer_nvfp4(64, 256), q.dense(), t4) == q.QDG_ERR_UNSUPPORTED
    pm = q.qdg_plan_create(q.layer_nvfp4(64, 256, num_experts=4), q.moe(2))
    assert "w4a16-nvfp4" in q.qdg_moe_describe(pm, 8, 16)
    # bf16 activations: no activation scales needed, none quantized here
    assert _status(q.qdg_quantize_act, q.layer_nvfp4(64, 256), 0x1000, 4, 0x2000, 0x3000, 0) == q.QDG_ERR_UNSUPPORTED
    # the per-tensor scale is required by preprocess; weights are not produced here
    layer = q.layer_nvfp4(100, 256)
    n = q.qdg_preprocess_query(layer)
    w = q.StdWeights(qweight=0x1000, scales=0x2000, zeros=None, tensor_scale=None)
    assert _status(q.qdg_preprocess, layer, w, 0x10000, n, 0) == q.QDG_ERR_INVALID_ARG
    # the producer needs a buffer for the tensor scales (passed as `zeros`)
    assert _status(q.qdg_quantize_weights, layer, 0x1000, 0x2000, 0x3000, None, 0) == q.QDG_ERR_INVALID_ARG
    # packed size: 1 KiB of codes and 128 bytes of scale records per 16 x 128 unit, plus the tensor scale
    units = 7 * 2
    assert n == ((units * 1024 + 255) // 256 * 256 + 256 + units * 128 + 255) // 256 * 256


def test_moe_128_row_blocks():
    # 128-row blocks (plain output only) run the LDS-tiled families: the bf16
    # one for NVFP4, W8A16 and W2A16, the 8-bit one for W8A8, W4A8,
    # W4A8-MXFP4, W4A4 and MXFP4 x INT8
    for layer, fam in ((q.layer_nvfp4(256, 256, num_experts=4), "tile"), (q.layer_w8a16(256, 256, num_experts=4), "tile"),
                       (q.layer_w2a16(256, 256, num_experts=4), "tile"),
                       (q.layer_w8a8(256, 256, num_experts=4), "qtile"), (q.layer_w4a8(256, 256, num_experts=4), "qtile"),
                       (q.layer_mxfp4(256, 256, num_experts=4), "qtile"), (q.layer_w4a4(256, 256, num_experts=4), "qtile"),
                       (q.layer_mxfp4_int8(256, 256, num_experts=4), "qtile")):
        p = q.qdg_plan_create(layer, q.moe(2))
        assert f"family={fam} " in q.qdg_moe_describe(p, 8, 128)
        # 64-row blocks: the 8-bit LDS-tiled family's 64 x 512 tiles
        assert ("family=qtile " if fam == "qtile" else "family=stream ") in q.qdg_moe_describe(p, 8, 64)
        ps = q.qdg_plan_create(layer, q.moe(2, epilogue=q.QDG_EPI_SILU_MUL))
        with pytest.raises(q.QdgError):
            q.qdg_moe_describe(ps, 8, 128)



def test_noalloc_refuses_oversized_workspace_before_device_work():
    # M = 8192 at K = 14336 with a 16-way K split needs GBs of partials: the
    # allocation-free entry point refuses it on the host (no pointer is used)
    layer = q.layer_w4a16(4096, 14336)
    plan = q.qdg_plan_create(layer, q.dense(), q.TuningConfig(block_m=128, split_k=16))
    assert q.qdg_plan_workspace(plan, 8192) > q.QDG_NOALLOC_SCRATCH_BYTES
    assert _status(q.qdg_gemm_noalloc, plan, None, None, None, None, 8192) == q.QDG_ERR_WORKSPACE
    assert "workspace" in q.qdg_last_error()
    assert q.load().qdg_gemm_noalloc(None, None, None, None, None, 16, None) == q.QDG_ERR_INVALID_ARG


def test_tuned_split_never_exceeds_the_k_groups():
    # K = 1024 holds 8 groups of 128: a tuning that asks for more splits gets
    # one group per split in every family (no empty K range is launched)
    cases = [(q.layer_w4a16(4096, 1024), q.TuningConfig(block_m=128, split_k=64), 256, "family=tile"),
             (q.layer_w8a8(4096, 1024), q.TuningConfig(block_m=128, split_k=64), 256, "family=qtile"),
             (q.layer_w8a8(4096, 1024), q.TuningConfig(block_m=32, block_n=32, split_k=64), 32, "family=stream"),
             (q.layer_w4a16(4096, 1024), q.TuningConfig(block_m=16, split_k=64), 16, "family=wstream")]
    for layer, tun, m, fam in cases:
        d = q.qdg_plan_describe(q.qdg_plan_create(layer, q.dense(), tun), m)
        assert fam in d and "split_k=8 " in d, d


def test_moe_padding_skip_choice():
    # 8-bit LDS-tiled MoE: the instance that skips all-padding 32-row halves
    # of blocks serves calls whose experts average at most one block of rows
    # (T*top_k <= E*block_m); the bf16 tiles skip inside every MoE instance
    E, top_k = 256, 8
    for mk in (q.layer_w8a8, q.layer_w4a8, q.layer_mxfp4, q.layer_w4a4, q.layer_mxfp4_int8):
        p = q.qdg_plan_create(mk(4096, 7168, num_experts=E), q.moe(top_k))
        for t, bm in ((512, 64), (2048, 64), (2049, 64), (4096, 64), (4096, 128), (4097, 128)):
            d = q.qdg_moe_describe(p, t, bm)
            assert "family=qtile " in d, d
            assert ("pad_skip=1" in d) == (t * top_k <= E * bm), (t, bm, d)
        assert "pad_skip" not in q.qdg_plan_describe(q.qdg_plan_create(mk(4096, 7168), q.dense()), 4096)
    pw = q.qdg_plan_create(q.layer_w4a16(4096, 7168, num_experts=E), q.moe(top_k))
    assert "pad_skip" not in q.qdg_moe_describe(pw, 512, 64)


def test_moe_16_row_tile_tuning():
    # block_n 512 names the 16 x 512 tiles of grouped W4A16 16-row blocks;
    # without a tuning they serve K <= 2048 (16 groups), the streaming family
    # longer K; other formats and dense plans reject the tuning
    big = q.layer_w4a16(4096, 7168, num_experts=256)
    short = q.layer_w4a16(7168, 2048, num_experts=256)
    t16 = q.TuningConfig(block_m=16, block_n=512, waves=8)
    assert "family=tile block_m=16 block_n=512" in q.qdg_moe_describe(q.qdg_plan_create(big, q.moe(8), t16), 64, 16)
    assert "family=stream block_m=16" in q.qdg_moe_describe(q.qdg_plan_create(big, q.moe(8)), 64, 16)
    assert "family=tile block_m=16 block_n=512" in q.qdg_moe_describe(q.qdg_plan_create(short, q.moe(8)), 64, 16)
    pin = q.TuningConfig(block_n=64, waves=4)
    assert "family=stream block_m=16" in q.qdg_moe_describe(q.qdg_plan_create(short, q.moe(8), pin), 64, 16)
    assert _status(q.qdg_plan_create, q.layer_w8a8(4096, 7168, num_experts=8), q.moe(8), t16) == q.QDG_ERR_UNSUPPORTED
    assert _status(q.qdg_plan_create, q.layer_w4a16(4096, 7168), q.dense(), t16) == q.QDG_ERR_UNSUPPORTED
    assert _status(q.qdg_plan_create, big, q.moe(8), q.TuningConfig(block_n=512, waves=4)) == q.QDG_ERR_UNSUPPORTED


def test_few_row_routing():
    # W4A16 up to 8 rows where weight streaming would split K: streaming
    # family; the 8-bit formats use weight streaming only for narrow layers
    # with at least 32 K groups, else the streaming family with one tile per
    # workgroup up to 512 tiles and no K split from 128 workgroups
    d = lambda layer, m: q.qdg_plan_describe(q.qdg_plan_create(layer, q.dense()), m)  # noqa: E731
    assert "family=stream block_m=16 block_n=32 split_k=4" in d(q.layer_w4a16(4096, 14336), 8)
    assert "family=wstream" in d(q.layer_w4a16(4096, 14336), 9)
    assert "family=wstream" in d(q.layer_w8a8(4096, 4096), 16)
    assert "family=stream block_m=16 block_n=32 split_k=1" in d(q.layer_w8a8(14336, 4096), 16)
    assert "family=stream block_m=16 block_n=16 split_k=1" in d(q.layer_mxfp4(7168, 2048), 16)
    assert "family=wstream" in d(q.layer_mxfp4(2048, 7168), 16)
    assert "family=stream block_m=16 block_n=64 split_k=1" in d(q.layer_w8a16(14336, 4096), 16)
