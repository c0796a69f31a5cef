"""Python binding of libqdg.so (fused dequantize-and-multiply GEMM for MI355X).

Argument marshalling only: every function forwards to the C entry point of the
same name in ``include/qdg.h``; all computation runs in the library's HIP
kernels. Pointers are plain integers (for example ``tensor.data_ptr()``) and
``stream`` is a HIP stream handle as an integer (0 = default stream;
``current_stream()`` returns torch's current one). A non-OK status raises
``QdgError`` carrying the library's message.

The library must have been built (``quantized_dequant_gemm_amd.build``); there
is no fallback of any kind when it is missing.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqdg.so")

# enums (mirror include/qdg.h)
QDG_OK, QDG_ERR_INVALID_ARG, QDG_ERR_UNSUPPORTED, QDG_ERR_MISALIGNED, QDG_ERR_WORKSPACE, QDG_ERR_HIP = range(6)
QDG_W_INT4, QDG_W_UINT4, QDG_W_INT8, QDG_W_MXFP4, QDG_W_NVFP4, QDG_W_UINT2 = range(6)
QDG_S_F16, QDG_S_F32, QDG_S_E8M0, QDG_S_E4M3 = range(4)
QDG_A_BF16, QDG_A_INT8, QDG_A_FP8E4M3, QDG_A_MXFP4 = range(4)
QDG_O_BF16, QDG_O_F32, QDG_O_I32 = range(3)
QDG_KIND_DENSE, QDG_KIND_MOE = range(2)
QDG_EPI_NONE, QDG_EPI_SILU_MUL = range(2)
QDG_FLAG_BAD_SCALE, QDG_FLAG_BAD_ZERO_POINT, QDG_FLAG_BAD_EXPERT_ID = 1, 2, 4

STATUS_NAMES = {0: "QDG_OK", 1: "QDG_ERR_INVALID_ARG", 2: "QDG_ERR_UNSUPPORTED", 3: "QDG_ERR_MISALIGNED",
                4: "QDG_ERR_WORKSPACE", 5: "QDG_ERR_HIP"}

# Every symbol include/qdg.h declares (the ABI test checks the list against the header).
EXPORTS = (
    "qdg_version", "qdg_last_error", "qdg_validate_layer", "qdg_preprocess_query", "qdg_preprocess",
    "qdg_quantize_weights", "qdg_quantize_act", "qdg_plan_create", "qdg_plan_destroy", "qdg_plan_workspace",
    "qdg_plan_describe", "qdg_moe_describe", "qdg_gemm", "qdg_moe_align_capacity", "qdg_moe_align",
    "qdg_moe_gemm", "qdg_moe_combine", "qdg_moe_combine_bf16", "qdg_plan_autotune", "qdg_plan_autotune_reset",
    "qdg_plan_jit", "qdg_gemm_noalloc",
)


class LayerConfig(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("k", ctypes.c_int64), ("num_experts", ctypes.c_int64),
                ("wtype", ctypes.c_int32), ("stype", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("has_zeros", ctypes.c_int32), ("atype", ctypes.c_int32), ("act_group", ctypes.c_int32),
                ("otype", ctypes.c_int32), ("arch", ctypes.c_int32)]


class ComputeConfig(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("batch_invariant", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("epilogue", ctypes.c_int32)]


class TuningConfig(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32), ("block_k", ctypes.c_int32),
                ("split_k", ctypes.c_int32), ("stages", ctypes.c_int32), ("waves", ctypes.c_int32),
                ("mfma", ctypes.c_int32), ("load_path", ctypes.c_int32)]


class StdWeights(ctypes.Structure):
    _fields_ = [("qweight", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("zeros", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_void_p)]


class QdgError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def load():
    """Load libqdg.so (raises OSError/RuntimeError if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run python -m quantized_dequant_gemm_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "qdg_version": (ctypes.c_char_p, []),
        "qdg_last_error": (ctypes.c_char_p, []),
        "qdg_validate_layer": (I32, [P]),
        "qdg_preprocess_query": (I32, [P, P]),
        "qdg_preprocess": (I32, [P, P, P, SZ, P, P]),
        "qdg_quantize_weights": (I32, [P, P, P, P, P, P]),
        "qdg_quantize_act": (I32, [P, P, I64, P, P, P]),
        "qdg_plan_create": (I32, [P, P, P, P]),
        "qdg_plan_destroy": (None, [P]),
        "qdg_plan_workspace": (I32, [P, I64, P]),
        "qdg_plan_describe": (ctypes.c_int, [P, I64, ctypes.c_char_p, SZ]),
        "qdg_moe_describe": (ctypes.c_int, [P, I64, I32, ctypes.c_char_p, SZ]),
        "qdg_gemm": (I32, [P, P, P, P, P, I64, P, SZ, P]),
        "qdg_gemm_noalloc": (I32, [P, P, P, P, P, I64, P]),
        "qdg_moe_align_capacity": (I32, [I64, I32, I32, I32, P]),
        "qdg_moe_align": (I32, [P, I64, I32, I32, I32, P, P, P, P, P]),
        "qdg_moe_gemm": (I32, [P, P, P, P, P, P, P, I64, I32, I32, P, P, SZ, P]),
        "qdg_moe_combine": (I32, [P, P, I64, I32, I64, P, I32, P]),
        "qdg_moe_combine_bf16": (I32, [P, P, I64, I32, I64, P, I32, P]),
        "qdg_plan_autotune": (I32, [P, P, P, P, P, I64, P, SZ, I32, P, P, P]),
        "qdg_plan_autotune_reset": (I32, [P]),
        "qdg_plan_jit": (I32, [P, I64, I32, ctypes.c_char_p, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status):
    if status != QDG_OK:
        raise QdgError(status, load().qdg_last_error().decode())


def _ref(x):
    return None if x is None else ctypes.byref(x)


def current_stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


# ------------------------------------------------------------- entry points

def qdg_version():
    return load().qdg_version().decode()


def qdg_last_error():
    return load().qdg_last_error().decode()


def qdg_validate_layer(layer):
    _check(load().qdg_validate_layer(ctypes.byref(layer)))


def qdg_preprocess_query(layer):
    out = ctypes.c_size_t()
    _check(load().qdg_preprocess_query(ctypes.byref(layer), ctypes.byref(out)))
    return out.value


def qdg_preprocess(layer, weights, packed, packed_bytes, stream=0, status=None):
    """status: optional device pointer to a caller-zeroed uint32 that receives QDG_FLAG_* bits."""
    _check(load().qdg_preprocess(ctypes.byref(layer), ctypes.byref(weights), packed, packed_bytes, status,
                                 stream))


def qdg_quantize_weights(layer, w, qweight, scales, zeros=None, stream=0):
    _check(load().qdg_quantize_weights(ctypes.byref(layer), w, qweight, scales, zeros, stream))


def qdg_quantize_act(layer, a_bf16, M, qa, a_scales, stream=0):
    _check(load().qdg_quantize_act(ctypes.byref(layer), a_bf16, M, qa, a_scales, stream))


class Plan:
    """Owns a qdg_plan* (destroyed with the object)."""

    def __init__(self, handle):
        self.handle = handle

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.qdg_plan_destroy(self.handle)
            self.handle = None


def qdg_plan_create(layer, compute, tuning=None):
    h = ctypes.c_void_p()
    _check(load().qdg_plan_create(ctypes.byref(layer), ctypes.byref(compute), _ref(tuning), ctypes.byref(h)))
    return Plan(h)


def qdg_plan_destroy(plan):
    if plan.handle:
        load().qdg_plan_destroy(plan.handle)
        plan.handle = None


def qdg_plan_workspace(plan, M):
    out = ctypes.c_size_t()
    _check(load().qdg_plan_workspace(plan.handle, M, ctypes.byref(out)))
    return out.value


def qdg_plan_describe(plan, M):
    n = load().qdg_plan_describe(plan.handle, M, None, 0)
    if n < 0:
        raise QdgError(QDG_ERR_INVALID_ARG, "describe failed")
    buf = ctypes.create_string_buffer(n + 1)
    load().qdg_plan_describe(plan.handle, M, buf, n + 1)
    return buf.value.decode()


def qdg_moe_describe(plan, T, block_m):
    n = load().qdg_moe_describe(plan.handle, T, block_m, None, 0)
    if n < 0:
        raise QdgError(QDG_ERR_INVALID_ARG, "describe failed (not a MoE plan or unsupported block_m)")
    buf = ctypes.create_string_buffer(n + 1)
    load().qdg_moe_describe(plan.handle, T, block_m, buf, n + 1)
    return buf.value.decode()


def qdg_gemm(plan, A, a_scales, packed, Y, M, workspace, ws_bytes, stream=0):
    _check(load().qdg_gemm(plan.handle, A, a_scales, packed, Y, M, workspace, ws_bytes, stream))


QDG_NOALLOC_SCRATCH_BYTES = 64 << 20


def qdg_gemm_noalloc(plan, A, a_scales, packed, Y, M, stream=0):
    """qdg_gemm on the library's own per-GPU scratch array (no workspace)."""
    _check(load().qdg_gemm_noalloc(plan.handle, A, a_scales, packed, Y, M, stream))


def qdg_moe_align_capacity(T, top_k, num_experts, block_m):
    out = ctypes.c_int64()
    _check(load().qdg_moe_align_capacity(T, top_k, num_experts, block_m, ctypes.byref(out)))
    return out.value


def qdg_moe_align(topk_ids, T, top_k, num_experts, block_m, sorted_ids, block_expert, num_padded, stream=0,
                  status=None):
    """status: optional device pointer to a caller-zeroed uint32 that receives QDG_FLAG_BAD_EXPERT_ID."""
    _check(load().qdg_moe_align(topk_ids, T, top_k, num_experts, block_m, sorted_ids, block_expert,
                                num_padded, status, stream))


def qdg_moe_gemm(plan, A, a_scales, packed, sorted_ids, block_expert, num_padded, T, block_m, a_per_pair, Y,
                 workspace, ws_bytes, stream=0):
    _check(load().qdg_moe_gemm(plan.handle, A, a_scales, packed, sorted_ids, block_expert, num_padded, T,
                               block_m, a_per_pair, Y, workspace, ws_bytes, stream))


def qdg_moe_combine(y, w, T, top_k, n, out, otype, stream=0):
    _check(load().qdg_moe_combine(y, w, T, top_k, n, out, otype, stream))


def qdg_moe_combine_bf16(y, w, T, top_k, n, out, otype, stream=0):
    _check(load().qdg_moe_combine_bf16(y, w, T, top_k, n, out, otype, stream))


def qdg_plan_autotune(plan, A, a_scales, packed, Y, M, workspace, ws_bytes, reps=10, stream=0):
    """Returns (chosen TuningConfig, best time per launch in us)."""
    chosen = TuningConfig()
    us = ctypes.c_float()
    _check(load().qdg_plan_autotune(plan.handle, A, a_scales, packed, Y, M, workspace, ws_bytes, reps, stream,
                                    ctypes.byref(chosen), ctypes.byref(us)))
    return chosen, us.value


class JitInfo(ctypes.Structure):
    _fields_ = [("compile_ms", ctypes.c_double), ("load_ms", ctypes.c_double), ("from_cache", ctypes.c_int32),
                ("code_bytes", ctypes.c_int32), ("key", ctypes.c_char * 32)]


def qdg_plan_jit(plan, M, block_m=0, cache_dir=None):
    """Returns the JitInfo of the run-time compiled instance serving M."""
    info = JitInfo()
    _check(load().qdg_plan_jit(plan.handle, M, block_m, cache_dir.encode() if cache_dir else None,
                               ctypes.byref(info)))
    return info


def qdg_plan_autotune_reset(plan):
    _check(load().qdg_plan_autotune_reset(plan.handle))


# ------------------------------------------------------------- config helpers

def layer_w4a16(n, k, asym=False, num_experts=1, otype=QDG_O_BF16):
    return LayerConfig(n=n, k=k, num_experts=num_experts, wtype=QDG_W_UINT4 if asym else QDG_W_INT4,
                       stype=QDG_S_F16, group_size=128, has_zeros=1 if asym else 0, atype=QDG_A_BF16,
                       act_group=0, otype=otype, arch=950)


def layer_w8a8(n, k, otype=QDG_O_BF16, num_experts=1):
    return LayerConfig(n=n, k=k, num_experts=num_experts, wtype=QDG_W_INT8, stype=QDG_S_F32, group_size=0, has_zeros=0,
                       atype=QDG_A_INT8, act_group=0, otype=otype, arch=950)


def layer_w4a8(n, k, otype=QDG_O_BF16, num_experts=1):
    return LayerConfig(n=n, k=k, num_experts=num_experts, wtype=QDG_W_INT4, stype=QDG_S_F16, group_size=128, has_zeros=0,
                       atype=QDG_A_INT8, act_group=0, otype=otype, arch=950)


def layer_mxfp4(n, k, otype=QDG_O_BF16, num_experts=1):
    return LayerConfig(n=n, k=k, num_experts=num_experts, wtype=QDG_W_MXFP4, stype=QDG_S_E8M0, group_size=32,
                       has_zeros=0, atype=QDG_A_FP8E4M3, act_group=128, otype=otype, arch=950)


def layer_w2a16(n, k, otype=QDG_O_BF16, num_experts=1):
    """2-bit asymmetric weights (uint2 codes, uint8 zero points, fp16 group-128 scales), bf16 activations."""
    return LayerConfig(n=n, k=k, num_experts=num_experts, wtype=QDG_W_UINT2, stype=QDG_S_F16, group_size=128,
                       has_zeros=1, atype=QDG_A_BF16, act_group=0, otype=otype, arch=950)


def layer_mxfp4_int8(n, k, otype=QDG_O_BF16, num_experts=1):
    """MXFP4 weights with per-token int8 activations (the MXFP4 -> INT8 path)."""
    return LayerConfig(n=n, k=k, num_experts=num_experts, wtype=QDG_W_MXFP4, stype=QDG_S_E8M0, group_size=32,
                       has_zeros=0, atype=QDG_A_INT8, act_group=0, otype=otype, arch=950)


def layer_w8a16(n, k, otype=QDG_O_BF16, num_experts=1):
    """int8 weights with fp32 per-channel scales, bf16 activations."""
    return LayerConfig(n=n, k=k, num_experts=num_experts, wtype=QDG_W_INT8, stype=QDG_S_F32, group_size=0,
                       has_zeros=0, atype=QDG_A_BF16, act_group=0, otype=otype, arch=950)


def layer_nvfp4(n, k, otype=QDG_O_BF16, num_experts=1):
    """NVFP4 weights (E2M1, E4M3 scale per 16 K, fp32 scale per tensor) with
    bf16 activations."""
    return LayerConfig(n=n, k=k, num_experts=num_experts, wtype=QDG_W_NVFP4, stype=QDG_S_E4M3, group_size=16,
                       has_zeros=0, atype=QDG_A_BF16, act_group=0, otype=otype, arch=950)


def layer_w4a4(n, k, otype=QDG_O_BF16, num_experts=1):
    """MXFP4 weights with MXFP4 activations (E8M0 per 32-block on both sides)."""
    return LayerConfig(n=n, k=k, num_experts=num_experts, wtype=QDG_W_MXFP4, stype=QDG_S_E8M0, group_size=32,
                       has_zeros=0, atype=QDG_A_MXFP4, act_group=32, otype=otype, arch=950)


def dense(batch_invariant=0):
    return ComputeConfig(kind=QDG_KIND_DENSE, batch_invariant=batch_invariant, top_k=0, epilogue=QDG_EPI_NONE)


def moe(top_k, batch_invariant=0, epilogue=0):
    return ComputeConfig(kind=QDG_KIND_MOE, batch_invariant=batch_invariant, top_k=top_k, epilogue=epilogue)
