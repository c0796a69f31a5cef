"""Helpers for the GPU parity tests: standard-format tensors from oracle data,
and one call of each library entry point through the C ABI binding.

Inputs come from ``synth`` (seeded draws) and the oracle's quantizers; the
library only ever sees device copies of them.
"""

import numpy as np
import torch

import quantized_dequant_gemm_amd as q
from oracle import codecs


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def bf16_dev(bits):
    return dev(np.asarray(bits, np.uint16).view(np.int16), torch.bfloat16)


def to_f64(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def assert_elementwise(y, y64):
    """Per-element bound beside the Frobenius one, for every compared output:
    |y - y64| <= 2^-8 |y64| + 2^-10 rms(row of y64). Rounding an fp32 result
    to bf16 (RNE) moves it by at most 2^-9 of itself, so the first term holds
    the output rounding with a factor 2 to spare (for fp32 outputs it only
    loosens the bound); the second holds the fp32 accumulation of the kernel,
    which is orders of magnitude below it, while a wrong element (a dropped
    group, a swapped column, a stale value) is off by about the row's rms."""
    y = np.atleast_2d(to_f64(y) if isinstance(y, torch.Tensor) else np.asarray(y, np.float64))
    y64 = np.atleast_2d(np.asarray(y64, np.float64))
    assert y.shape == y64.shape, (y.shape, y64.shape)
    rms = np.sqrt(np.mean(y64 * y64, axis=1, keepdims=True))
    bound = 2.0 ** -8 * np.abs(y64) + 2.0 ** -10 * rms
    bad = np.argwhere(~(np.abs(y - y64) <= bound))
    assert bad.size == 0, [(int(r), int(c), y[r, c], y64[r, c], bound[r, c]) for r, c in bad[:6]]


def workspace(plan, m):
    nbytes = q.qdg_plan_workspace(plan, m)
    return torch.zeros(nbytes, dtype=torch.uint8, device="cuda"), nbytes


def out_tensor(m, n, otype):
    dt = {q.QDG_O_BF16: torch.bfloat16, q.QDG_O_F32: torch.float32, q.QDG_O_I32: torch.int32}[otype]
    return torch.full((m, n), float("nan") if dt != torch.int32 else -(2 ** 31), dtype=dt, device="cuda")


class Packed:
    """A layer in the kernel layout (keeps its device buffers alive)."""

    def __init__(self, layer, qweight, scales, zeros=None, tensor_scale=None):
        self.layer = layer
        self.std = (qweight, scales, zeros, tensor_scale)
        self.nbytes = q.qdg_preprocess_query(layer)
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device="cuda")
        w = q.StdWeights(qweight=qweight.data_ptr(), scales=scales.data_ptr(),
                         zeros=zeros.data_ptr() if zeros is not None else None,
                         tensor_scale=tensor_scale.data_ptr() if tensor_scale is not None else None)
        q.qdg_preprocess(layer, w, self.buf.data_ptr(), self.nbytes, q.current_stream())


def std_w4(q_vals, s16, zeros=None):
    """Signed int4 values (zeros None) or unsigned codes (with zeros) -> device std tensors."""
    codes = codecs.encode_int4(q_vals) if zeros is None else np.asarray(q_vals, np.uint8)
    qw = dev(codecs.pack_nibbles(codes))
    sc = dev(np.asarray(s16, np.uint16).view(np.int16))
    z = dev(np.asarray(zeros, np.uint8)) if zeros is not None else None
    return qw, sc, z


def gemm(layer, packed, a_dev, m, a_scales=None, compute=None, tuning=None, y=None):
    plan = q.qdg_plan_create(layer, compute or q.dense(), tuning)
    ws, nbytes = workspace(plan, m)
    if y is None:
        y = out_tensor(m, layer.n, layer.otype)
    q.qdg_gemm(plan, a_dev.data_ptr(), a_scales.data_ptr() if a_scales is not None else None,
               packed.buf.data_ptr(), y.data_ptr(), m, ws.data_ptr(), nbytes, q.current_stream())
    torch.cuda.synchronize()
    return y, plan


def w4a16(a_bits, q_vals, s16, zeros=None, otype=q.QDG_O_BF16, compute=None, tuning=None):
    n, k = np.asarray(q_vals).shape
    layer = q.layer_w4a16(n, k, asym=zeros is not None, otype=otype)
    qw, sc, z = std_w4(q_vals, s16, zeros)
    pk = Packed(layer, qw, sc, z)
    a = bf16_dev(a_bits)
    y, _ = gemm(layer, pk, a, a.shape[0], compute=compute, tuning=tuning)
    return y
