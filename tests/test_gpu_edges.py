"""Edge codes and bad input at the GPU boundary.

1. The extreme codes of the standard format -- int4 -8 (nibble 0x8) and int8
   -128 -- through every kernel family that serves them, compared exactly
   with the oracle: one-hot activations with fp32 output for the bf16-
   activation paths (each output is one dequantized weight, exact in fp32),
   the raw int32 accumulator for the int8-activation paths (int8 activation
   codes also reach -128 there). The oracle's own quantizers never emit these
   codes (their ranges are [-7, 7] and [-127, 127]), so the codes are drawn
   directly.
2. The input flags of qdg_preprocess and qdg_moe_align: each forbidden value
   (E8M0 255, E4M3 NaN, non-finite f16 / f32 scale, UINT4 zero above 15,
   expert id outside [0, E)) sets its bit in the caller's status word, and
   clean input leaves the word zero.
"""

import numpy as np
import pytest
import torch

import quantized_dequant_gemm_amd as q
from oracle import codecs, ref
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _family(plan, m):
    return q.qdg_plan_describe(plan, m).split("family=")[1].split()[0]


def _int4_codes(n, k, seed):
    """int4 values in [-8, 7] with -8 in every (column, 128-group)."""
    r = np.random.default_rng(seed)
    v = r.integers(-8, 8, size=(n, k))
    v[:, 5::128] = -8
    v[:, 77::128] = 7
    return v


def _int8_codes(shape, seed):
    """int8 values in [-128, 127] with -128 in every row."""
    r = np.random.default_rng(seed)
    v = r.integers(-128, 128, size=shape)
    v[..., 3] = -128
    return v


def _f16_pow2_scales(n, groups, seed):
    r = np.random.default_rng(seed)
    return codecs.f32_to_f16_bits(np.ldexp(1.0, r.integers(-12, -3, size=(n, groups))).astype(np.float32))


def _one_hot_sweep(run, k, m):
    """Calls run(a_bits) with m one-hot rows at a time until every k was hit;
    returns Y^T stacked as [k][n] (row i = the output of the row e_i)."""
    outs = []
    for base in range(0, k, m):
        ks = np.arange(base, base + m) % k
        a = np.zeros((m, k), np.float32)
        a[np.arange(m), ks] = 1.0
        y = H.to_f64(run(codecs.f32_to_bf16_bits(a)))
        outs.append(y[: min(m, k - base)])
    return np.concatenate(outs)


# -------------------------------------------------- W4A16: int4 code -8

@pytest.mark.parametrize("m,family", [(16, "wstream"), (32, "stream"), (64, "tile")])
def test_w4a16_int4_minus8_one_hot(qdg, m, family):
    k, n = 384, 96
    v = _int4_codes(n, k, seed=m)
    s = _f16_pow2_scales(n, k // 128, seed=m + 1)
    w64 = ref.dequant_int4_sym(v, s)
    layer = q.layer_w4a16(n, k, otype=q.QDG_O_F32)
    qw, sc, _ = H.std_w4(v, s)
    pk = H.Packed(layer, qw, sc)
    plan = q.qdg_plan_create(layer, q.dense())
    assert _family(plan, m) == family

    def run(a_bits):
        return H.gemm(layer, pk, H.bf16_dev(a_bits), m)[0]
    got = _one_hot_sweep(run, k, m)
    assert np.array_equal(got, w64.T)


# ------------------------------------- W4A8 / W8A8: int4 -8, int8 -128 (raw int32)

@pytest.mark.parametrize("m,family", [(16, "wstream"), (16, "stream"), (40, "stream"), (160, "qtile")])
@pytest.mark.parametrize("kind", ["w4a8", "w8a8"])
def test_int8_paths_extreme_codes_raw_exact(qdg, kind, m, family):
    # (K = 512 is short: 16 rows stream by default, weight streaming is
    # pinned by a tuning)
    k, n = 512, 272
    qa = _int8_codes((m, k), seed=m + 7)
    if kind == "w4a8":
        v = _int4_codes(n, k, seed=m + 3)
        s = _f16_pow2_scales(n, k // 128, seed=m)
        qw, sc, _ = H.std_w4(v, s)
        layer = q.layer_w4a8(n, k, otype=q.QDG_O_I32)
    else:
        v = _int8_codes((n, k), seed=m + 3)
        qw = H.dev(v.astype(np.int8))
        sc = H.dev(np.full(n, 0.5, np.float32))
        layer = q.layer_w8a8(n, k, otype=q.QDG_O_I32)
    pk = H.Packed(layer, qw, sc)
    plan = q.qdg_plan_create(layer, q.dense())
    tuning = (q.TuningConfig(block_m=128) if family == "qtile" else
              q.TuningConfig(waves=8) if family == "wstream" else None)
    if tuning is None:
        assert _family(plan, m) == family
    y, plan_used = H.gemm(layer, pk, H.dev(qa.astype(np.int8)), m, tuning=tuning)
    assert _family(plan_used, m) == family
    assert np.array_equal(y.cpu().numpy().astype(np.int64), ref.int_matmul(qa, v))


# ------------------------------------------------- W8A16: int8 -128, one-hot

@pytest.mark.parametrize("m,family", [(16, "stream"), (64, "tile")])
def test_w8a16_int8_minus128_one_hot(qdg, m, family):
    k, n = 384, 80
    v = _int8_codes((n, k), seed=m + 11)
    sw = np.ldexp(1.0, np.random.default_rng(m).integers(-10, -2, n)).astype(np.float32)
    layer = q.layer_w8a16(n, k, otype=q.QDG_O_F32)
    pk = H.Packed(layer, H.dev(v.astype(np.int8)), H.dev(sw))
    plan = q.qdg_plan_create(layer, q.dense())
    assert _family(plan, m) == family

    def run(a_bits):
        return H.gemm(layer, pk, H.bf16_dev(a_bits), m)[0]
    got = _one_hot_sweep(run, k, m)
    assert np.array_equal(got, (v.astype(np.float64) * sw[:, None]).T)


# ------------------------------------------------------------- grouped MoE

def _align(ids, E, bm):
    t, top_k = ids.shape
    cap = q.qdg_moe_align_capacity(t, top_k, E, bm)
    sid = torch.empty(cap, dtype=torch.int32, device="cuda")
    blk = torch.empty(cap // bm, dtype=torch.int32, device="cuda")
    npad = torch.zeros(1, dtype=torch.int32, device="cuda")
    q.qdg_moe_align(H.dev(ids.astype(np.int32)).data_ptr(), t, top_k, E, bm, sid.data_ptr(), blk.data_ptr(),
                    npad.data_ptr(), q.current_stream())
    return sid, blk, npad


def _moe_run(layer, pk, a_dev, a_scales, ids, bm, a_per_pair, tuning=None):
    t, top_k = ids.shape
    sid, blk, npad = _align(ids, layer.num_experts, bm)
    plan = q.qdg_plan_create(layer, q.moe(top_k), tuning)
    ws, nbytes = H.workspace(plan, t)
    y = H.out_tensor(t * top_k, layer.n, layer.otype)
    q.qdg_moe_gemm(plan, a_dev.data_ptr(), a_scales.data_ptr() if a_scales is not None else None,
                   pk.buf.data_ptr(), sid.data_ptr(), blk.data_ptr(), npad.data_ptr(), t, bm, a_per_pair,
                   y.data_ptr(), ws.data_ptr(), nbytes, q.current_stream())
    torch.cuda.synchronize()
    return y, q.qdg_moe_describe(plan, t, bm)


@pytest.mark.parametrize("bm,stream", [(16, False), (16, True), (32, False), (64, False), (128, False)])
def test_moe_w4a16_int4_minus8_one_hot(qdg, bm, stream):
    # token t's row is e_{k_t}; each of its top-2 pair rows is then one
    # column of its expert's dequantized weight, exact in fp32 (16-row
    # blocks of this short K run the LDS-tiled family, or the streaming one
    # when a tuning pins it)
    E, top_k, k, n, t = 3, 2, 256, 64, 150
    vs = [_int4_codes(n, k, seed=50 + e) for e in range(E)]
    ss = [_f16_pow2_scales(n, k // 128, seed=60 + e) for e in range(E)]
    layer = q.layer_w4a16(n, k, num_experts=E, otype=q.QDG_O_F32)
    qw = H.dev(np.stack([codecs.pack_nibbles(codecs.encode_int4(v)) for v in vs]))
    sc = H.dev(np.stack(ss).view(np.int16))
    pk = H.Packed(layer, qw, sc)
    r = np.random.default_rng(bm)
    ids = np.stack([r.permutation(E)[:top_k] for _ in range(t)]).astype(np.int32)
    kt = r.integers(0, k, t)
    a = np.zeros((t, k), np.float32)
    a[np.arange(t), kt] = 1.0
    tun = q.TuningConfig(block_n=64, waves=4) if stream else None
    y, desc = _moe_run(layer, pk, H.bf16_dev(codecs.f32_to_bf16_bits(a)), None, ids, bm, 0, tuning=tun)
    assert ("family=stream " if stream else "family=tile ") in desc
    want = np.stack([ref.dequant_int4_sym(vs[ids[p // top_k, p % top_k]], ss[ids[p // top_k, p % top_k]])[:, kt[p // top_k]]
                     for p in range(t * top_k)])
    assert np.array_equal(H.to_f64(y), want)


@pytest.mark.parametrize("bm", [16, 32, 64, 128])
@pytest.mark.parametrize("kind", ["w4a8", "w8a8"])
def test_moe_int8_extreme_codes_raw_exact(qdg, kind, bm):
    E, top_k, k, n, t = 3, 2, 256, 96, 90
    r = np.random.default_rng(bm + 1)
    ids = np.stack([r.permutation(E)[:top_k] for _ in range(t)]).astype(np.int32)
    h = _int8_codes((t * top_k, k), seed=bm + 5)  # per-pair input (down projection)
    if kind == "w4a8":
        vs = [_int4_codes(n, k, seed=70 + e) for e in range(E)]
        ss = [_f16_pow2_scales(n, k // 128, seed=80 + e) for e in range(E)]
        layer = q.layer_w4a8(n, k, num_experts=E, otype=q.QDG_O_I32)
        pk = H.Packed(layer, H.dev(np.stack([codecs.pack_nibbles(codecs.encode_int4(v)) for v in vs])),
                      H.dev(np.stack(ss).view(np.int16)))
    else:
        vs = [_int8_codes((n, k), seed=90 + e) for e in range(E)]
        layer = q.layer_w8a8(n, k, num_experts=E, otype=q.QDG_O_I32)
        pk = H.Packed(layer, H.dev(np.stack(vs).astype(np.int8)), H.dev(np.full((E, n), 0.25, np.float32)))
    y, desc = _moe_run(layer, pk, H.dev(h.astype(np.int8)), None, ids, bm, 1)
    assert ("family=qtile " if bm in (64, 128) else "family=stream ") in desc
    flat = ids.reshape(-1)
    want = np.stack([ref.int_matmul(h[p:p + 1], vs[flat[p]])[0] for p in range(t * top_k)])
    assert np.array_equal(y.cpu().numpy().astype(np.int64), want)


@pytest.mark.parametrize("bm", [16, 128])
def test_moe_w8a16_int8_minus128_one_hot(qdg, bm):
    E, top_k, k, n, t = 2, 1, 256, 64, 200
    vs = [_int8_codes((n, k), seed=100 + e) for e in range(E)]
    sws = [np.ldexp(1.0, np.random.default_rng(110 + e).integers(-10, -2, n)).astype(np.float32) for e in range(E)]
    layer = q.layer_w8a16(n, k, num_experts=E, otype=q.QDG_O_F32)
    pk = H.Packed(layer, H.dev(np.stack(vs).astype(np.int8)), H.dev(np.stack(sws)))
    r = np.random.default_rng(bm + 2)
    ids = r.integers(0, E, (t, top_k)).astype(np.int32)
    kt = r.integers(0, k, t)
    a = np.zeros((t, k), np.float32)
    a[np.arange(t), kt] = 1.0
    y, desc = _moe_run(layer, pk, H.bf16_dev(codecs.f32_to_bf16_bits(a)), None, ids, bm, 0)
    assert ("family=tile" in desc) == (bm == 128)
    want = np.stack([vs[ids[i, 0]][:, kt[i]].astype(np.float64) * sws[ids[i, 0]] for i in range(t)])
    assert np.array_equal(H.to_f64(y), want)


# ----------------------------------------------------------- input flags

def _status_word():
    return torch.zeros(1, dtype=torch.int32, device="cuda")


def _preprocess_status(layer, qw, sc, z=None, ts=None):
    st = _status_word()
    nbytes = q.qdg_preprocess_query(layer)
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    w = q.StdWeights(qw.data_ptr(), sc.data_ptr(), z.data_ptr() if z is not None else None,
                     ts.data_ptr() if ts is not None else None)
    q.qdg_preprocess(layer, w, buf.data_ptr(), nbytes, q.current_stream(), status=st.data_ptr())
    torch.cuda.synchronize()
    return int(st.item())


def test_flag_mxfp4_e8m0_255(qdg):
    n, k = 32, 256
    codes = np.random.default_rng(1).integers(0, 16, (n, k)).astype(np.uint8)
    e = np.full((n, k // 32), 120, np.uint8)
    layer = q.layer_mxfp4(n, k)
    qw = H.dev(codecs.pack_nibbles(codes))
    assert _preprocess_status(layer, qw, H.dev(e)) == 0
    e[17, 3] = 255
    assert _preprocess_status(layer, qw, H.dev(e)) == q.QDG_FLAG_BAD_SCALE


def test_flag_nvfp4_e4m3_nan_and_tensor_scale(qdg):
    n, k = 32, 256
    codes = np.random.default_rng(2).integers(0, 16, (n, k)).astype(np.uint8)
    sb = np.full((n, k // 16), 0x38, np.uint8)
    layer = q.layer_nvfp4(n, k)
    qw = H.dev(codecs.pack_nibbles(codes))
    ts = H.dev(np.array([0.5], np.float32))
    assert _preprocess_status(layer, qw, H.dev(sb), ts=ts) == 0
    for bad in (0x7F, 0xFF):
        sb2 = sb.copy()
        sb2[5, 9] = bad
        assert _preprocess_status(layer, qw, H.dev(sb2), ts=ts) == q.QDG_FLAG_BAD_SCALE
    assert _preprocess_status(layer, qw, H.dev(sb), ts=H.dev(np.array([np.inf], np.float32))) == q.QDG_FLAG_BAD_SCALE


def test_flag_int4_f16_scale_and_uint4_zero(qdg):
    n, k = 48, 256
    v = _int4_codes(n, k, seed=3)
    s = _f16_pow2_scales(n, k // 128, seed=4)
    layer = q.layer_w4a16(n, k)
    qw, sc, _ = H.std_w4(v, s)
    assert _preprocess_status(layer, qw, sc) == 0
    s2 = s.copy()
    s2[7, 1] = 0x7C00  # +inf
    assert _preprocess_status(layer, qw, H.dev(s2.view(np.int16))) == q.QDG_FLAG_BAD_SCALE
    s2[7, 1] = 0x7E00  # NaN
    assert _preprocess_status(q.layer_w4a8(n, k), qw, H.dev(s2.view(np.int16))) == q.QDG_FLAG_BAD_SCALE
    codes = np.random.default_rng(5).integers(0, 16, (n, k)).astype(np.uint8)
    z = np.full((n, k // 128), 8, np.uint8)
    la = q.layer_w4a16(n, k, asym=True)
    qa_, sa_, za = H.std_w4(codes, s, z)
    assert _preprocess_status(la, qa_, sa_, za) == 0
    z[40, 0] = 16
    assert _preprocess_status(la, qa_, sa_, H.dev(z)) == q.QDG_FLAG_BAD_ZERO_POINT


def test_flag_int8_channel_scale(qdg):
    n, k = 40, 256
    v = _int8_codes((n, k), seed=6)
    sw = np.full(n, 0.01, np.float32)
    for mk in (q.layer_w8a8, q.layer_w8a16):
        layer = mk(n, k)
        assert _preprocess_status(layer, H.dev(v.astype(np.int8)), H.dev(sw)) == 0
        sw2 = sw.copy()
        sw2[33] = np.nan
        assert _preprocess_status(layer, H.dev(v.astype(np.int8)), H.dev(sw2)) == q.QDG_FLAG_BAD_SCALE


@pytest.mark.parametrize("bm", [16, 128])
def test_flag_moe_align_bad_expert_id(qdg, bm):
    E, top_k, t = 8, 2, 100
    r = np.random.default_rng(bm)
    ids = np.stack([r.permutation(E)[:top_k] for _ in range(t)]).astype(np.int32)
    cap = q.qdg_moe_align_capacity(t, top_k, E, bm)

    def run(ids):
        st = _status_word()
        sid = torch.empty(cap, dtype=torch.int32, device="cuda")
        blk = torch.empty(cap // bm, dtype=torch.int32, device="cuda")
        npad = torch.zeros(1, dtype=torch.int32, device="cuda")
        q.qdg_moe_align(H.dev(ids).data_ptr(), t, top_k, E, bm, sid.data_ptr(), blk.data_ptr(), npad.data_ptr(),
                        q.current_stream(), status=st.data_ptr())
        torch.cuda.synchronize()
        n = int(npad.item())
        return int(st.item()), sid.cpu().numpy()[:n], blk.cpu().numpy()[:n // bm]

    st, sid, blk = run(ids)
    assert st == 0
    bad = ids.copy()
    bad[3, 1] = E
    bad[60, 0] = -1
    st, sid, blk = run(bad)
    assert st == q.QDG_FLAG_BAD_EXPERT_ID
    # the other pairs are sorted exactly as the oracle sorts them (it keeps
    # only ids in [0, E)); the two bad pairs appear nowhere
    r_sid, r_blk, _ = ref.moe_align(bad, E, bm)
    assert np.array_equal(sid, r_sid) and np.array_equal(blk, r_blk)
    assert 3 * top_k + 1 not in sid and 60 * top_k not in sid
