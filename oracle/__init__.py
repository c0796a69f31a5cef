"""CPU fp64 oracle for the fused dequantize-and-multiply GEMM.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, obviously-correct
definition that the HIP library is checked against. Only the test suite, the
smoke check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may
import it. The library (``quantized_dequant_gemm_amd``) never imports, links or
calls anything here, and nothing here imports the library: the two share no
code. The only module both sides use is ``synth`` (seeded random draws, no
arithmetic of the method).

What the pages fix and what they leave open
-------------------------------------------
The pages (the Humming release as covered by retrivium.ai, jetabc.cn and
kinachrichten.com) name the ingredients of a quantized weight -- integer or
floating 4-bit codes, scales per group or per block, zero points, symmetric or
asymmetric quantization (jetabc, section on what quantization is; kinachrichten,
"Warum quantisierte Kernel wichtig sind") -- and say that every export format is
brought into one standard form of weights, scales and zero points before a
kernel repacks it ("Wie die Architektur funktioniert"). They print no formula,
no layout and no worked example. The readings taken here:

* dequantization is affine per contiguous K-group: ``w = (q - z) * s`` with an
  integer zero point ``z`` in the code domain (``z = 0`` when symmetric);
* a linear layer's weight is stored ``[N, K]`` and ``Y = A @ deq(W).T``;
* MXFP4, FP8 E4M3 and E8M0 follow the OCP Microscaling v1.0 and OCP 8-bit
  floating point specifications; bf16 is the top half of IEEE binary32;
* every rounding is IEEE round-to-nearest-even.

Modules
-------
``codecs``  exact decoders (code -> real) and RNE encoders for each storage type
``quant``   producers of the standard format (weights) and activation quantizers
``ref``     dequantize-then-matmul references, MoE routing and the expert sort
``metrics`` comparison helpers

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, brute force, library routines or the specifications'
own definitions; none is "parity unpinned".
"""

from . import codecs, quant, ref, metrics  # noqa: F401
