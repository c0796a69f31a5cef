"""Seeded synthetic inputs shared by the oracle-side tests and the HIP path.

This module only draws random numbers and casts them to storage types with
library casts; it holds none of the arithmetic of the dequantize-and-multiply
method (no quantizer, no dequantizer, no GEMM). Both the oracle and the
library consume what it returns, so it is the one piece they share.

Recipe (workloads of the pages' kind -- dense and MoE linear layers of a large
language model, kinachrichten "Warum quantisierte Kernel wichtig sind"; the
pages publish no dataset or tensor statistics, so all values are synthetic):

* base seed 20261021; per tensor ``seed = base + 100 * workload_id + tensor_id``
  with tensor ids A=1, W=2, router logits=3, MoE hidden H=4 (numpy PCG64);
* activations ``A ~ N(0, 1)`` drawn in float64, cast to float32, then to bf16
  with torch's round-to-nearest-even cast;
* weights ``W ~ N(0, 0.02)`` in float32 (quantized afterwards by whichever side
  needs the standard format);
* router logits ``~ N(0, 1)`` float64 ``[T, E]``; the MoE down-projection input
  ``H ~ N(0, 1)`` bf16 ``[T * top_k, intermediate]``.

Workload ids: 0 tiny W4A16, 1 dense W4A16, 2 W8A8/W4A8, 3 W4A8-MXFP4, 4 MoE.
"""

import numpy as np

BASE_SEED = 20261021
TID_A, TID_W, TID_LOGITS, TID_H = 1, 2, 3, 4


def seed_for(workload_id, tensor_id, salt=0):
    return BASE_SEED + 100 * workload_id + tensor_id + 100000 * salt


def rng(workload_id, tensor_id, salt=0):
    return np.random.Generator(np.random.PCG64(seed_for(workload_id, tensor_id, salt)))


def normal_f32(shape, std, workload_id, tensor_id, salt=0):
    g = rng(workload_id, tensor_id, salt)
    return (g.standard_normal(shape) * std).astype(np.float32)


def activations_bf16_bits(m, k, workload_id, salt=0, tensor_id=TID_A):
    """A ~ N(0,1) as bf16 bit patterns (uint16 [m, k]) via torch's RNE cast."""
    import torch
    x = normal_f32((m, k), 1.0, workload_id, tensor_id, salt)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def weights_f32(n, k, workload_id, salt=0):
    """W ~ N(0, 0.02) float32 [n, k]."""
    return normal_f32((n, k), 0.02, workload_id, TID_W, salt)


def router_logits(t, e, workload_id=4, salt=0):
    return rng(workload_id, TID_LOGITS, salt).standard_normal((t, e))


def moe_hidden_bf16_bits(rows, k, workload_id=4, salt=0):
    return activations_bf16_bits(rows, k, workload_id, salt, tensor_id=TID_H)


# ----------------------------------------------------------- device draws
# Large inputs for timing runs (GB-sized expert weights) are drawn on the
# device with torch's seeded generator instead of numpy; same distributions.


def device_normal_f32(shape, std, seed, device="cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def device_activations_bf16(m, k, seed, device="cuda"):
    import torch
    return device_normal_f32((m, k), 1.0, seed, device).to(torch.bfloat16)
