"""Dequantize-then-matmul references in float64, MoE routing and expert sort.

Test infrastructure (see the package docstring).

The computation is exact arithmetic done fast, so the reference is its plain
definition: decode every stored code to its real value in float64, form the
dequantized weight matrix, multiply with float64 BLAS.

* Affine per-group dequantization ``w = (q - z) * s`` (readings in the package
  docstring; the pages list scales, zero points, group size and
  symmetric/asymmetric schemes -- kinachrichten, "Warum quantisierte Kernel
  wichtig sind").
* The integer paths (W8A8, W4A8) are products of integer-valued matrices whose
  partial sums stay far below 2**53, so float64 BLAS returns them exactly
  whatever its summation order; ``int_matmul`` also offers an int64 path.
* The grouped MoE GEMM applies, for every (token, slot) pair, the GEMM of the
  expert it was routed to (jetabc, "跑得有多快", names the grouped MoE path;
  kinachrichten, "Warum quantisierte Kernel wichtig sind", motivates MoE).
"""

import numpy as np

from . import codecs


# ---------------------------------------------------------------- dequant


def dequant_int4_sym(codes_or_vals, scales_f16_bits, group=128):
    """Signed values q [N,K] (ints in [-8,7]) and fp16 scales [N,K/G] -> W64."""
    q = np.asarray(codes_or_vals).astype(np.float64)
    s = codecs.f16_bits_to_f64(scales_f16_bits)
    n, k = q.shape
    return (q.reshape(n, k // group, group) * s[:, :, None]).reshape(n, k)


def dequant_uint4_asym(q, scales_f16_bits, zeros, group=128):
    """Unsigned codes q [N,K] in [0,15], fp16 scales and uint8 zero points [N,K/G]."""
    q = np.asarray(q).astype(np.float64)
    s = codecs.f16_bits_to_f64(scales_f16_bits)
    z = np.asarray(zeros).astype(np.float64)
    n, k = q.shape
    w = (q.reshape(n, k // group, group) - z[:, :, None]) * s[:, :, None]
    return w.reshape(n, k)


def dequant_uint2_asym(q, scales_f16_bits, zeros, group=128):
    """2-bit codes q [N,K] in [0,3], fp16 scales and uint8 zero points
    [N,K/G] -> W64 = (q - z) * s per group (the affine rule of the 4-bit
    codes; the pages list WNA16 widths without fixing them: kinachrichten,
    "Warum quantisierte Kernel wichtig sind")."""
    q = np.asarray(q).astype(np.int64)
    assert np.all((q >= 0) & (q <= 3)), "2-bit codes are 0..3"
    z = np.asarray(zeros).astype(np.int64)
    assert np.all(z <= 3), "2-bit zero points are 0..3"
    s = codecs.f16_bits_to_f64(scales_f16_bits)
    n, k = q.shape
    w = (q.reshape(n, k // group, group) - z[:, :, None]).astype(np.float64) * s[:, :, None]
    return w.reshape(n, k)


def dequant_mxfp4(codes, e8m0, block=32):
    """E2M1 codes [N,K] and E8M0 scale codes [N,K/32] -> W64."""
    e = np.asarray(e8m0)
    assert not np.any(e == 255), "E8M0 code 255 is NaN and not a valid scale"
    v = codecs.decode_e2m1(codes)
    s = codecs.decode_e8m0(e)
    n, k = v.shape
    return (v.reshape(n, k // block, block) * s[:, :, None]).reshape(n, k)


def dequant_nvfp4(codes, e4m3, tensor_scale, block=16):
    """E2M1 codes [N,K], E4M3 scale codes [N,K/16] and the binary32 tensor
    scale -> W64 = e2m1(q) * e4m3(s) * ts (NVFP4: a 4-bit floating format
    the pages name beside INT4, kinachrichten, "Warum quantisierte Kernel
    wichtig sind")."""
    sc = codecs.decode_e4m3(e4m3)
    assert not np.any(np.isnan(sc)), "E4M3 NaN codes are not valid scales"
    v = codecs.decode_e2m1(codes)
    n, k = v.shape
    w = v.reshape(n, k // block, block) * sc[:, :, None] * float(np.float32(tensor_scale))
    return w.reshape(n, k)


# ---------------------------------------------------------------- GEMMs


def int_matmul(a, b_t):
    """Exact integer product ``a @ b_t.T`` (int64; independent of BLAS)."""
    return np.asarray(a).astype(np.int64) @ np.asarray(b_t).astype(np.int64).T


def gemm_w4a16(a_bf16_bits, w64):
    """Y64 = A @ W.T for bf16 activations [M,K] and dequantized W64 [N,K]."""
    a = codecs.bf16_bits_to_f64(a_bf16_bits)
    return a @ np.asarray(w64, dtype=np.float64).T


def gemm_w8a8(qa, sa, qw, sw):
    """Per-token int8 activations times per-channel int8 weights.

    Returns (Y64 [M,N], P int64 [M,N]) with ``Y = sa[m] * sw[n] * P`` and
    ``P = sum_k qa[m,k] * qw[n,k]`` the exact int32-range accumulator.
    """
    p = np.asarray(qa, dtype=np.float64) @ np.asarray(qw, dtype=np.float64).T
    y = p * np.asarray(sa, np.float64)[:, None] * np.asarray(sw, np.float64)[None, :]
    return y, p.astype(np.int64)


def gemm_w8a16(a_bf16_bits, qw, sw):
    """bf16 activations times per-channel int8 weights (W8A16, a WNA16 width
    the pages list): ``Y = A @ (q * s).T`` with the dequantized weights
    ``w[n,k] = q[n,k] * s[n]`` in float64."""
    a = codecs.bf16_bits_to_f64(a_bf16_bits)
    w = np.asarray(qw, np.float64) * np.asarray(sw, np.float64)[:, None]
    return a @ w.T


def gemm_w4a8(qa, sa, q_int4_vals, sw_f16_bits, group=128):
    """Per-token int8 activations times int4 weights with fp16 group scales.

    Returns (Y64, P_total int64) where
    ``Y[m,n] = sa[m] * sum_g sw[n,g] * sum_{k in g} qa[m,k] * q[n,k]`` and
    ``P_total = sum_k qa[m,k] * q[n,k]`` (the accumulator with unit scales).
    """
    qa = np.asarray(qa, dtype=np.float64)
    q = np.asarray(q_int4_vals, dtype=np.float64)
    sw = codecs.f16_bits_to_f64(sw_f16_bits)
    m, k = qa.shape
    n = q.shape[0]
    y = np.zeros((m, n))
    for g in range(k // group):
        sl = slice(g * group, (g + 1) * group)
        y += (qa[:, sl] @ q[:, sl].T) * sw[None, :, g]
    y *= np.asarray(sa, np.float64)[:, None]
    p = (qa @ q.T).astype(np.int64)
    return y, p


def dequant_act_fp8(codes, sa, group=128):
    """E4M3 activation codes [M,K] with fp32 scales [M,K/group] -> A64."""
    v = codecs.decode_e4m3(codes)
    assert not np.any(np.isnan(v)), "E4M3 NaN code in activations"
    m, k = v.shape
    s = np.asarray(sa, np.float64)
    return (v.reshape(m, k // group, group) * s[:, :, None]).reshape(m, k)


def gemm_mxfp4(a_codes, sa, w_codes, w_e8m0):
    """fp8 E4M3 activations (per token-group-128 scales) times MXFP4 weights."""
    a = dequant_act_fp8(a_codes, sa)
    w = dequant_mxfp4(w_codes, w_e8m0)
    return a @ w.T


def gemm_mxfp4_int8(qa, sa, w_codes, w_e8m0):
    """Per-token int8 activations times MXFP4 weights (the pages' MXFP4 ->
    INT8 path, kinachrichten, "Das Wichtigste in Kürze" and "Kompilierzeiten
    und gerätespezifisches Tuning"): ``Y[m,n] = sa[m] * sum_k qa[m,k] *
    w[n,k]`` with ``w = e2m1(q) * 2**(E - 127)`` per 32-block, in float64.
    Every product qa * e2m1 * 2**(E-127) is a short dyadic number, so the
    float64 sum of a row is exact whenever its terms' exponents stay within
    53 bits of each other (always, for the block scales of quantized
    weights)."""
    a = np.asarray(qa, np.float64)
    w = dequant_mxfp4(w_codes, w_e8m0)
    return (a @ w.T) * np.asarray(sa, np.float64)[:, None]


def gemm_w4a4(a_codes, a_e8m0, w_codes, w_e8m0):
    """MXFP4 activations times MXFP4 weights (W4A4): both sides decoded with
    their E8M0 block-32 scales, then a float64 product."""
    a = dequant_mxfp4(a_codes, a_e8m0)
    w = dequant_mxfp4(w_codes, w_e8m0)
    return a @ w.T


def gemm_nvfp4a16(a_bf16_bits, codes, e4m3, tensor_scale):
    """bf16 activations times NVFP4 weights: ``Y = A @ W64.T`` with the
    weights dequantized in float64."""
    return codecs.bf16_bits_to_f64(a_bf16_bits) @ dequant_nvfp4(codes, e4m3, tensor_scale).T


def dequant_act_int8(qa, sa):
    return np.asarray(qa, np.float64) * np.asarray(sa, np.float64)[:, None]


# ---------------------------------------------------------------- MoE


def route_topk(logits, top_k):
    """Softmax over experts in float64, then the top_k experts per token.

    Order: descending probability, ties to the lower expert id. Returns
    (ids int32 [T, top_k], probs float64 [T, top_k]).
    """
    x = np.asarray(logits, dtype=np.float64)
    x = x - x.max(axis=1, keepdims=True)
    p = np.exp(x)
    p /= p.sum(axis=1, keepdims=True)
    # stable argsort on (-p) keeps the lower id first among equal values
    order = np.argsort(-p, axis=1, kind="stable")[:, :top_k]
    return order.astype(np.int32), np.take_along_axis(p, order, axis=1)


def moe_align(topk_ids, num_experts, block_m):
    """Sort (token, slot) pairs by expert and pad each expert to block_m rows.

    Flat pair index ``i = t * top_k + j``. Within an expert the pairs keep
    ascending flat order. Each expert's segment is padded up to a multiple of
    ``block_m`` with the sentinel ``T * top_k``; experts without pairs get no
    block. Returns (sorted_ids int32 [num_padded], block_expert int32
    [num_padded / block_m], num_padded).
    """
    ids = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    total = ids.size
    sorted_ids = []
    block_expert = []
    for e in range(num_experts):
        members = list(np.nonzero(ids == e)[0])  # ascending flat order
        if not members:
            continue
        nblk = -(-len(members) // block_m)
        seg = list(members) + [total] * (nblk * block_m - len(members))
        sorted_ids.extend(seg)
        block_expert.extend([e] * nblk)
    return (np.asarray(sorted_ids, dtype=np.int32),
            np.asarray(block_expert, dtype=np.int32), len(sorted_ids))


def moe_gemm_rows(a_rows_bf16_bits, topk_ids, expert_w64, input_is_per_pair):
    """Reference output of the grouped GEMM for every (token, slot) pair.

    ``expert_w64(e)`` returns expert e's dequantized weight [N, K] in float64
    (dequantizing one expert at a time keeps memory bounded).
    Gate+up: row ``t*top_k+j`` of the output is ``X[t] @ W_e.T``.
    Down: ``input_is_per_pair`` -- the input row is ``H[t*top_k+j]``.
    Returns Y64 [T*top_k, N].
    """
    ids = np.asarray(topk_ids)
    t_count, top_k = ids.shape
    a = codecs.bf16_bits_to_f64(a_rows_bf16_bits)
    flat = ids.reshape(-1)
    y = None
    for e in np.unique(flat):
        pairs = np.nonzero(flat == e)[0]
        rows = pairs if input_is_per_pair else pairs // top_k
        w = expert_w64(int(e))
        ye = a[rows] @ w.T
        if y is None:
            y = np.zeros((flat.size, w.shape[0]))
        y[pairs] = ye
    return y


def moe_rows(topk_ids, input_is_per_pair, expert_rows_ref):
    """The grouped GEMM of any format: for every (token, slot) pair, the dense
    reference of the expert it was routed to, on the pair's input row.

    ``expert_rows_ref(e, rows)`` returns expert e's dense reference on the
    activation rows ``rows`` (token rows for gate+up, pair rows for down):
    either Y64 [len(rows), N] or (Y64, P) with P the exact integer
    accumulator of the integer formats. Returns Y64 [T*top_k, N], and P int64
    [T*top_k, N] when the reference gives one (else None).
    """
    ids = np.asarray(topk_ids)
    top_k = ids.shape[1]
    flat = ids.reshape(-1)
    y = p = None
    for e in np.unique(flat):
        pairs = np.nonzero(flat == e)[0]
        rows = pairs if input_is_per_pair else pairs // top_k
        r = expert_rows_ref(int(e), rows)
        ye, pe = r if isinstance(r, tuple) else (r, None)
        if y is None:
            y = np.zeros((flat.size, ye.shape[1]))
            if pe is not None:
                p = np.zeros((flat.size, ye.shape[1]), dtype=np.int64)
        y[pairs] = ye
        if pe is not None:
            p[pairs] = pe
    return y, p


# ---------------------------------------------------------------- MoE block

def silu_mul(y_gate_up):
    """The gate+up epilogue: Y [R, 2I] holds the gate projection in columns
    [0, I) and the up projection in [I, 2I); returns H [R, I] with
    ``H = silu(G) * U`` and ``silu(x) = x * sigmoid(x) = x / (1 + exp(-x))``
    in float64 (the MoE block around the grouped GEMM; jetabc, "跑得有多快")."""
    y = np.asarray(y_gate_up, dtype=np.float64)
    i = y.shape[1] // 2
    g, u = y[:, :i], y[:, i:]
    # x * sigmoid(x) with the sigmoid in the form that cannot overflow
    e = np.exp(-np.abs(g))
    sig = np.where(g >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return g * sig * u


def moe_combine(y_pairs, route_w, top_k):
    """The top-k weighted combine: ``out[t] = sum_j w[t, j] * Y[t*top_k + j]``
    over the grouped GEMM's pair rows, in float64."""
    y = np.asarray(y_pairs, dtype=np.float64)
    w = np.asarray(route_w, dtype=np.float64).reshape(-1, top_k)
    t = w.shape[0]
    return np.einsum("tj,tjc->tc", w, y.reshape(t, top_k, -1))
