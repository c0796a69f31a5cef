"""Write the oracle regression fixtures in this folder (calls only oracle/ and synth).

The pages print no worked example, so these fixtures freeze the oracle's own
answer on the tiny asymmetric W4A16 workload (A bf16 [16,1024] ~ N(0,1);
W f32 [512,1024] ~ N(0,0.02) -> uint4, group 128, fp16 scales, uint8 zeros)
and on a small MoE expert sort, so that any later change to the oracle's
arithmetic shows up as a diff that its commit has to justify.

Run: python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import synth  # noqa: E402
from oracle import quant, ref  # noqa: E402


def sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def tiny_w4a16():
    a = synth.activations_bf16_bits(16, 1024, workload_id=0)
    w = synth.weights_f32(512, 1024, workload_id=0)
    q, s, z = quant.quantize_uint4_asym(w)
    y = ref.gemm_w4a16(a, ref.dequant_uint4_asym(q, s, z))
    pick = [(0, 0), (3, 17), (15, 511), (7, 256), (12, 100)]
    return {
        "workload": "tiny W4A16 asym uint4 g128: M16 K1024 N512",
        "sha256_codes": sha(q.astype(np.uint8)),
        "sha256_scales_f16": sha(s),
        "sha256_zeros": sha(z),
        "y64_samples": [[i, j, float(y[i, j])] for i, j in pick],
        "y64_frobenius": float(np.linalg.norm(y)),
    }


def small_moe_align():
    ids, _ = ref.route_topk(synth.router_logits(64, 256), 8)
    sid, blk, npad = ref.moe_align(ids, 256, 16)
    return {
        "workload": "MoE sort: T64 top8 E256 block_m16",
        "sha256_topk_ids": sha(ids.astype(np.int32)),
        "sha256_sorted_ids": sha(sid), "sha256_block_expert": sha(blk),
        "num_padded": int(npad),
    }


if __name__ == "__main__":
    out = {"tiny_w4a16": tiny_w4a16(), "moe_align_t64": small_moe_align()}
    with open(os.path.join(HERE, "oracle_regression.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))
