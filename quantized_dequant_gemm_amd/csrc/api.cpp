// C ABI of libqdg.so: validation, plans (kernel-instance selection per M
// range), workspace accounting and launches. See include/qdg.h.
//
// The split follows the pages: the standard format says what the stored
// values mean, the Layer/Compute/Tuning configs and the per-device heuristics
// decide how a given M is executed (kinachrichten, "Wie die Architektur
// funktioniert"). Unsupported combinations are rejected with a message, and
// qdg_plan_describe reports which instance serves which M ("vLLM Humming: why
// shared quantization still needs specialized kernels", sections
// "Specialization should leave a reproducible trail" and "The architectural
// gain is a smaller maintenance surface").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "qdg_internal.h"

using namespace qdg;

namespace {

thread_local std::string g_last_error;

qdg_status fail(qdg_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

qdg_status ok() { return QDG_OK; }

qdg_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return QDG_OK;
  return fail(QDG_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr size_t kCounterBytes = 64 * 1024;
constexpr int kTargetWorkgroups = 512;  // two 4-wave workgroups per CU (256 CUs)
constexpr int kWsTargetWorkgroups = 256;  // weight streaming: one workgroup per CU

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

}  // namespace

namespace qdg {

qdg_status report_error(qdg_status st, const char* msg) { return fail(st, "%s", msg); }

Format format_of(const qdg_layer_config& L) {
  if (L.wtype == QDG_W_INT8) return L.atype == QDG_A_BF16 ? FMT_W8A16 : FMT_W8A8;
  if (L.wtype == QDG_W_MXFP4)
    return L.atype == QDG_A_MXFP4 ? FMT_W4A4 : L.atype == QDG_A_INT8 ? FMT_MXFP4_I8 : FMT_MXFP4;
  if (L.wtype == QDG_W_NVFP4) return FMT_NVFP4;
  if (L.wtype == QDG_W_UINT2) return FMT_W2A16;
  if (L.atype == QDG_A_INT8) return FMT_W4A8;
  return FMT_W4A16;
}

PackedGeom packed_geom(const qdg_layer_config& L, Format f) {
  PackedGeom g;
  g.n = L.n;
  g.k = L.k;
  g.n_pad = align_up(L.n, 16);
  g.ntiles = g.n_pad / 16;
  g.groups = L.k / 128;
  g.experts = L.num_experts;
  const int64_t units = g.ntiles * g.groups;
  g.w_bytes = units * (f == FMT_W8A8 || f == FMT_W8A16 ? 2048 : f == FMT_W2A16 ? 512 : 1024);  // per 16x128 unit
  switch (f) {
    case FMT_W4A16:
    case FMT_W2A16: g.s_bytes = units * 16 * 8; break;  // {f32 s, bf16x2 -(128+z)}
    case FMT_W4A8: g.s_bytes = units * 16 * 4; break;   // f32 s/16
    case FMT_MXFP4:
    case FMT_MXFP4_I8:
    case FMT_W4A4: g.s_bytes = units * 64; break;       // E8M0 per lane
    case FMT_W8A8:
    case FMT_W8A16: g.s_bytes = g.n_pad * 4; break;     // f32 per column
    case FMT_NVFP4: g.s_bytes = 256 + units * 128; break;  // f32 tensor scale, then 2 E4M3 per lane
  }
  g.s_offset = align_up(g.w_bytes, 256);
  g.expert_stride = align_up(g.s_offset + g.s_bytes, 256);
  return g;
}

}  // namespace qdg

// One autotuned M range: M in (2^(b-1), 2^b] for entry b (entry 0: M = 1).
struct AutoEntry {
  bool valid;
  qdg_tuning_config tuning;
  float us;
};
constexpr int kAutoRanges = 32;

// A run-time compiled streaming-family instance the plan launches instead of
// the ahead-of-time one (qdg_plan_jit).
struct JitInstance {
  int mt, nt, kw, device;  // streaming family: the instance's shape
  bool moe;
  hipFunction_t fn;
  std::string expr;  // other families: the kernel's name expression (empty for streaming instances)
};

struct qdg_plan {
  qdg_layer_config layer;
  qdg_compute_config compute;
  qdg_tuning_config tuning;
  bool has_tuning;
  Format fmt;
  PackedGeom geom;
  AutoEntry autot[kAutoRanges];  // written by qdg_plan_autotune only
  std::vector<JitInstance> jit;  // written by qdg_plan_jit only
};

namespace {

const char* fmt_name(Format f, const qdg_layer_config& L) {
  switch (f) {
    case FMT_W4A16: return L.wtype == QDG_W_UINT4 ? "w4a16-uint4-asym" : "w4a16-int4-sym";
    case FMT_W8A8: return "w8a8-int8";
    case FMT_W8A16: return "w8a16-int8";
    case FMT_W4A8: return "w4a8-int8";
    case FMT_MXFP4: return "w4a8-mxfp4-fp8";
    case FMT_W4A4: return "w4a4-mxfp4";
    case FMT_MXFP4_I8: return "w4a8-mxfp4-int8";
    case FMT_W2A16: return "w2a16-uint2-asym";
    case FMT_NVFP4: return "w4a16-nvfp4";
  }
  return "?";
}

qdg_status validate_layer(const qdg_layer_config* L) {
  if (!L) return fail(QDG_ERR_INVALID_ARG, "layer config is NULL");
  if (L->n < 1 || L->k < 1 || L->num_experts < 1)
    return fail(QDG_ERR_INVALID_ARG, "n, k and num_experts must be positive (n=%lld k=%lld E=%lld)",
                (long long)L->n, (long long)L->k, (long long)L->num_experts);
  if (L->arch != 950) return fail(QDG_ERR_UNSUPPORTED, "arch %d: only gfx950 (950) is built", L->arch);
  if (L->k % 128 != 0)
    return fail(QDG_ERR_UNSUPPORTED, "k=%lld is not a multiple of 128 (K is never padded)", (long long)L->k);
  if (L->n > (int64_t)1 << 26 || L->k > (int64_t)1 << 24)
    return fail(QDG_ERR_UNSUPPORTED, "n or k too large for the 32-bit tile indexing");
  if (L->otype < QDG_O_BF16 || L->otype > QDG_O_I32) return fail(QDG_ERR_INVALID_ARG, "bad otype %d", L->otype);
  switch (L->wtype) {
    case QDG_W_INT4:
    case QDG_W_UINT4: {
      if (L->stype != QDG_S_F16) return fail(QDG_ERR_UNSUPPORTED, "4-bit integer weights need f16 group scales");
      if (L->group_size != 128)
        return fail(QDG_ERR_UNSUPPORTED, "group_size %d: only 128 is implemented", L->group_size);
      const bool asym = L->wtype == QDG_W_UINT4;
      if (L->has_zeros != (asym ? 1 : 0))
        return fail(QDG_ERR_INVALID_ARG, "has_zeros must be %d for %s", asym ? 1 : 0, asym ? "UINT4" : "INT4");
      if (L->atype == QDG_A_BF16) {
        if (L->otype == QDG_O_I32) return fail(QDG_ERR_UNSUPPORTED, "W4A16 has no integer accumulator to return");
        return ok();
      }
      if (L->atype == QDG_A_INT8) {
        if (L->k > 65536) return fail(QDG_ERR_UNSUPPORTED, "int8 paths keep 16*|q*qa| sums in int32: k <= 65536");
        if (asym) return fail(QDG_ERR_UNSUPPORTED, "W4A8 with asymmetric uint4 weights is not implemented");
        if (L->act_group != 0) return fail(QDG_ERR_UNSUPPORTED, "W4A8 uses per-token activation scales (act_group 0)");
        return ok();
      }
      return fail(QDG_ERR_UNSUPPORTED, "4-bit integer weights with activation type %d", L->atype);
    }
    case QDG_W_INT8:
      if (L->stype != QDG_S_F32) return fail(QDG_ERR_UNSUPPORTED, "int8 weights need f32 per-channel scales");
      if (L->group_size != 0) return fail(QDG_ERR_UNSUPPORTED, "int8 weights are per channel (group_size 0)");
      if (L->has_zeros) return fail(QDG_ERR_UNSUPPORTED, "int8 weights are symmetric");
      if (L->atype == QDG_A_BF16) {  // W8A16
        if (L->act_group != 0) return fail(QDG_ERR_INVALID_ARG, "bf16 activations have no groups");
        if (L->otype == QDG_O_I32) return fail(QDG_ERR_UNSUPPORTED, "W8A16 has no integer accumulator");
        return ok();
      }
      if (L->atype != QDG_A_INT8 || L->act_group != 0)
        return fail(QDG_ERR_UNSUPPORTED, "int8 weights run with per-token int8 or bf16 activations");
      if (L->k > 65536) return fail(QDG_ERR_UNSUPPORTED, "int8 paths keep |q*qa| sums in int32: k <= 65536");
      return ok();
    case QDG_W_MXFP4:
      if (L->stype != QDG_S_E8M0 || L->group_size != 32)
        return fail(QDG_ERR_UNSUPPORTED, "MXFP4 needs E8M0 scales over blocks of 32");
      if (L->has_zeros) return fail(QDG_ERR_UNSUPPORTED, "MXFP4 has no zero points");
      if (!(L->atype == QDG_A_FP8E4M3 && L->act_group == 128) && !(L->atype == QDG_A_MXFP4 && L->act_group == 32) &&
          !(L->atype == QDG_A_INT8 && L->act_group == 0))
        return fail(QDG_ERR_UNSUPPORTED,
                    "MXFP4 weights run with fp8 E4M3 activations (128-group scales), MXFP4 activations (32-blocks) "
                    "or per-token int8 activations");
      if (L->otype == QDG_O_I32) return fail(QDG_ERR_UNSUPPORTED, "MXFP4 has no integer accumulator");
      return ok();
    case QDG_W_UINT2:
      if (L->stype != QDG_S_F16 || L->group_size != 128)
        return fail(QDG_ERR_UNSUPPORTED, "UINT2 weights need f16 scales over groups of 128");
      if (!L->has_zeros) return fail(QDG_ERR_INVALID_ARG, "UINT2 weights are asymmetric (has_zeros 1)");
      if (L->atype != QDG_A_BF16 || L->act_group != 0)
        return fail(QDG_ERR_UNSUPPORTED, "UINT2 weights run with bf16 activations");
      if (L->otype == QDG_O_I32) return fail(QDG_ERR_UNSUPPORTED, "W2A16 has no integer accumulator");
      return ok();
    case QDG_W_NVFP4:
      if (L->stype != QDG_S_E4M3 || L->group_size != 16)
        return fail(QDG_ERR_UNSUPPORTED, "NVFP4 needs E4M3 scales over blocks of 16");
      if (L->has_zeros) return fail(QDG_ERR_UNSUPPORTED, "NVFP4 has no zero points");
      if (L->atype != QDG_A_BF16 || L->act_group != 0)
        return fail(QDG_ERR_UNSUPPORTED, "NVFP4 weights run with bf16 activations");
      if (L->otype == QDG_O_I32) return fail(QDG_ERR_UNSUPPORTED, "NVFP4 has no integer accumulator");
      return ok();
    default:
      return fail(QDG_ERR_INVALID_ARG, "bad wtype %d", L->wtype);
  }
}

struct Choice {
  bool autotuned;  // served by an autotuned entry of the plan
  bool tile;
  bool ws;     // weight-streaming family (dense M <= 16, MoE 16-row blocks)
  bool qtile;  // LDS-tiled family of the 8-bit-activation formats
  StreamCfg sc;
  TileCfg tc;
  int grid_m;
  size_t partial_bytes;
  size_t rowsum_bytes;
  bool pad_skip;  // 8-bit LDS-tiled MoE: the instance that skips all-padding halves of blocks
};

// Device heuristics per M range for gfx950 (256 CUs): small M streams the
// weights with split-K to give every CU work; large M uses LDS-tiled MFMA.
Choice choose_t(const qdg_plan& P, int64_t M, const qdg_tuning_config& T, bool has_tuning) {
  Choice ch{};
  const PackedGeom& g = P.geom;
  const bool moe = P.compute.kind == QDG_KIND_MOE;
  int bm = has_tuning && T.block_m ? T.block_m : 0;
  if (!bm) bm = M <= 16 ? 16 : M <= 32 ? 32 : M <= 64 ? 64 : 128;
  // measured on MI355X: one (partly filled) 128-row block of the tiled
  // families, with K split into one pass of workgroups, beats the streaming
  // family from M = 33 (bf16 activations: W4A16, NVFP4, W8A16, W2A16) and
  // from M = 64 (int8 / fp8 / fp4 activations)
  const bool bf16_act = P.fmt == FMT_W4A16 || P.fmt == FMT_NVFP4 || P.fmt == FMT_W8A16 || P.fmt == FMT_W2A16;
  // W2A16 and MXFP4 weights with int8 activations have no weight-streaming
  // variant (the streaming family serves their small M)
  const bool no_wstream = P.fmt == FMT_MXFP4_I8 || P.fmt == FMT_W2A16;
  if (!has_tuning && !P.compute.batch_invariant && !moe && bm < 128 && M > (bf16_act ? 32 : 63))
    bm = 128;
  if (P.compute.batch_invariant && bm > 64) bm = 64;
  // the tiled family addresses A with 32-bit byte offsets
  const bool a_fits = (double)(M > 0 ? M : 1) * (double)g.k * 2.0 < 4294967296.0;
  // W4A16 with 33 to 64 rows: 64 x 512 tiles instead of one partly filled
  // 128-row block (a tuning asks for them with block_m 64 and block_n 512)
  const bool tile64 = P.fmt == FMT_W4A16 && !moe && !P.compute.batch_invariant &&
                      (has_tuning ? T.block_m == 64 && T.block_n == 512 : M > 32 && M <= 64);
  if ((bm >= 128 || tile64) &&
      (P.fmt == FMT_W4A16 || P.fmt == FMT_NVFP4 || P.fmt == FMT_W8A16 || P.fmt == FMT_W2A16) && !moe && a_fits) {
    // LDS-tiled family: BM x BN tiles, row sums of A per group in the workspace
    if (tile64) bm = 64;
    ch.tile = true;
    ch.tc.bm = bm;
    ch.tc.bn = bm == 256 ? 128 : bm == 64 ? 512 : 256;
    ch.tc.waves = tile64 ? 8 : has_tuning && T.waves ? T.waves : 8;
    ch.grid_m = (int)((M + bm - 1) / bm);
    const int64_t n_blocks = (g.ntiles + ch.tc.bn / 16 - 1) / (ch.tc.bn / 16);
    const int64_t tiles = n_blocks * ch.grid_m;
    // split K when the tiles alone leave CUs idle (fixed order: deterministic,
    // and independent of M only through the tile count)
    int split = has_tuning && T.split_k ? T.split_k : 0;
    if (!split) {
      // as many K splits as keep the workgroups within one pass over the CUs
      split = tiles >= 256 ? 1 : (int)(256 / tiles);
      const int maxs = (int)(g.groups / 2);
      if (split > maxs) split = maxs > 0 ? maxs : 1;
      if (split > 16) split = 16;
    }
    // a tuning's split beyond the group count would leave empty K ranges
    if (split > g.groups) split = (int)g.groups;
    ch.sc = StreamCfg{bm / 16, ch.tc.bn / 16, ch.tc.waves, split};
    ch.partial_bytes = split > 1 ? (size_t)tiles * split * ch.tc.bm * ch.tc.bn * 4 : 0;
    ch.rowsum_bytes = P.fmt == FMT_NVFP4 ? 0 : (size_t)ch.grid_m * bm * g.groups * 4;  // NVFP4: no offsets
    return ch;
  }
  // weight-streaming family: W4A16 with M <= 16, unless the caller pins a
  // streaming-family shape or asks for batch invariance (whose results must
  // not depend on which family a given M selects)
  const bool ws_tuning_ok =
      !has_tuning || ((!T.block_m || T.block_m == 16) && (!T.block_n || T.block_n == 64) && (!T.waves || T.waves == 8));
  // measured on MI355X (K = 14336, N = 4096, where weight streaming splits K
  // four ways): up to 8 rows the streaming family (two tiles per workgroup,
  // its own K split) is faster, 11.4 / 12.3 / 13.3 us at M = 1 / 4 / 8
  // against 13.4 / 13.5 / 14.0 us; at 16 rows both take 13.7 us
  const bool ws_split_few_rows =
      !has_tuning && !moe && M <= 8 && kWsTargetWorkgroups / ((g.ntiles + 3) / 4) > 1;
  if (bm == 16 && P.fmt == FMT_W4A16 && !P.compute.batch_invariant && ws_tuning_ok && !ws_split_few_rows &&
      (!moe || P.layer.wtype == QDG_W_INT4)) {
    ch.ws = true;
    ch.grid_m = 1;
    const int64_t nblocks = (g.ntiles + 3) / 4;
    int split = has_tuning && T.split_k ? T.split_k : (int)(kWsTargetWorkgroups / nblocks);
    if (moe || split < 1) split = 1;
    if (split > g.groups) split = (int)g.groups;
    ch.sc = StreamCfg{1, 4, 8, split};  // 16 x 64 per workgroup of 8 waves
    ch.partial_bytes = split > 1 ? (size_t)split * 16 * g.ntiles * 16 * 4 : 0;
    return ch;
  }
  // weight-streaming family of the int8 / fp8 formats (dense M <= 16): the
  // K range of a workgroup must fit its LDS; raw int32 output is not split
  // Without a tuning only narrow layers (one N tile per workgroup) with at
  // least 32 K groups stream this way: measured on MI355X at M = 16, W4A8
  // (K = 4096, N = 4096) 6.3 us against 7.0 us in the streaming family and
  // W4A8-MXFP4 (7168, 2048) 6.3 against 8.2 us, but W8A8 / W4A8 at
  // N = 14336 (4 tiles per workgroup) 16.8 / 11.3 against 15.3 / 10.2 us and
  // W4A8-MXFP4 (2048, 7168) (16 groups) 9.8 against 5.4 us
  const bool ws8_heuristic_ok = has_tuning || ((g.ntiles + 3) / 4 < 128 && g.groups >= 32);
  if (bm == 16 && P.fmt != FMT_W4A16 && P.fmt != FMT_W4A4 && P.fmt != FMT_W8A16 && P.fmt != FMT_NVFP4 && !moe &&
      !no_wstream &&
      !P.compute.batch_invariant &&
      ws_tuning_ok && ws8_heuristic_ok) {
    // 4 N tiles per workgroup when that gives enough workgroups, else one
    // tile with all 8 waves on its K range (no split across workgroups)
    const int nt = (g.ntiles + 3) / 4 >= 128 ? 4 : 1;
    const int64_t nblocks = (g.ntiles + nt - 1) / nt;
    const int min_split = (int)((g.groups + wstream8_max_groups() - 1) / wstream8_max_groups());
    int split = has_tuning && T.split_k ? T.split_k : (nblocks >= 128 ? 1 : (int)(kWsTargetWorkgroups / nblocks));
    if (split < min_split) split = min_split;
    if (split < 1) split = 1;
    if (split > g.groups) split = (int)g.groups;
    if (P.layer.otype == QDG_O_I32) split = min_split;
    if (P.layer.otype != QDG_O_I32 || split == 1) {
      ch.ws = true;
      ch.grid_m = 1;
      ch.sc = StreamCfg{1, nt, 8, split};
      ch.partial_bytes = split > 1 ? (size_t)split * 16 * g.ntiles * 16 * 4 : 0;
      return ch;
    }
  }
  // LDS-tiled family of the int8 / fp8 formats: 128 x 256 tiles, used once
  // there are enough of them (or M >= 512) to beat the streaming family
  const bool a8_fits =
      (double)(M > 0 ? M : 1) * (double)g.k * (P.fmt == FMT_MXFP4_I8 ? 2.0 : 1.0) < 4294967296.0;  // I8: two planes
  const int64_t q_tiles = ((M + 127) / 128) * ((g.ntiles + 15) / 16);
  // (measured on MI355X: from M = 64 the tiled family with K split into one
  // pass of 256 workgroups beats the streaming family at these layer sizes,
  // except where the streaming family's cheaper unit still wins up to 128
  // rows: fp4 x fp4 always, and int8 x int8 while the streaming grid of
  // 64 x 32 blocks is small enough to need a K split of its own)
  bool stream_mid = false;
  if (!has_tuning && M <= 128) {
    const int64_t stream_wgs = ((g.ntiles + 1) / 2) * ((M + 63) / 64);
    stream_mid = P.fmt == FMT_W4A4 || (P.fmt == FMT_W8A8 && 2 * stream_wgs <= kTargetWorkgroups);
  }
  const bool q_enough = (has_tuning && T.block_m >= 128) || (M >= 64 && !stream_mid);
  if (bm >= 128 && P.fmt != FMT_W4A16 && P.fmt != FMT_W8A16 && P.fmt != FMT_NVFP4 && P.fmt != FMT_W2A16 && !moe &&
      a8_fits && q_enough) {
    ch.tile = true;
    ch.qtile = true;
    ch.tc = TileCfg{128, 256, 8};
    ch.grid_m = (int)((M + 127) / 128);
    const int64_t n_blocks = (g.ntiles + 15) / 16;
    const int64_t tiles = n_blocks * ch.grid_m;
    int split = has_tuning && T.split_k ? T.split_k : 0;
    if (!split) {
      // as many K splits as keep the workgroups within one pass over the CUs
      split = tiles >= 256 ? 1 : (int)(256 / tiles);
      const int maxs = (int)(g.groups / 2);
      if (split > maxs) split = maxs > 0 ? maxs : 1;
      if (split > 16) split = 16;
    }
    if (split > g.groups) split = (int)g.groups;  // no empty K ranges
    if (P.layer.otype == QDG_O_I32) split = 1;  // integer results are never split
    ch.sc = StreamCfg{8, 16, 8, split};
    ch.partial_bytes = split > 1 ? (size_t)tiles * split * 128 * 256 * 4 : 0;
    ch.rowsum_bytes = 0;
    return ch;
  }
  if (bm > 64) bm = 64;  // other formats: the streaming family serves every M
  ch.tile = false;
  ch.sc.mt = bm / 16;
  ch.sc.kw = has_tuning && T.waves ? T.waves : 4;
  int nt = has_tuning && T.block_n ? T.block_n / 16 : 0;
  // measured on MI355X: NVFP4 and W8A16 in 16-row blocks, where two tiles per
  // workgroup leave too few workgroups and need a K split (256 to 511 tiles),
  // run fastest with one N tile per workgroup and no split instead (their
  // unpack is VALU-heavy); wider layers keep two tiles and no split
  const bool one_tile = ch.sc.mt == 1 && !P.compute.batch_invariant && !moe && g.ntiles >= 256 &&
                        g.ntiles < 512 && (P.fmt == FMT_NVFP4 || (P.fmt == FMT_W8A16 && g.groups <= 64));
  // Up to 16 rows of the formats other than W4A16 (measured on MI355X at
  // M = 16 over tile counts 1, 2, 4 and K splits 1 to 8): one tile per
  // workgroup while the layer has at most 512 tiles, two beyond (W8A16,
  // whose unpack is VALU-heavy: four; 17.0 against 18.3 us at N = 14336), and no K
  // split once that gives 128 workgroups (e.g. W4A4 (2048, 7168) 5.1 us
  // against 7.8 us for two tiles and two splits, W2A16 (4096, 4096) 7.2
  // against 8.9 us for two tiles and four splits): the split's extra
  // reduction launch costs more than the idle CUs
  const bool few_rows = ch.sc.mt == 1 && !P.compute.batch_invariant && !moe && P.fmt != FMT_W4A16;
  if (!nt && few_rows) nt = g.ntiles <= 512 ? 1 : P.fmt == FMT_W8A16 ? 4 : 2;
  if (!nt) nt = one_tile || (ch.sc.mt == 1 && g.ntiles < 128 && !P.compute.batch_invariant) ? 1 : 2;
  ch.sc.nt = nt;
  ch.grid_m = (int)((M + bm - 1) / bm);
  const int64_t nblocks = (g.ntiles + nt - 1) / nt;
  int split = has_tuning && T.split_k ? T.split_k : 0;
  if (!split && few_rows && nblocks >= 128) split = 1;
  if (!split) {
    const int64_t wgs = nblocks * (P.compute.batch_invariant ? 1 : ch.grid_m);
    split = (int)(kTargetWorkgroups / (wgs > 0 ? wgs : 1));
    if (split < 1) split = 1;
    const int maxs = (int)(g.groups / ch.sc.kw);
    if (split > maxs) split = maxs > 0 ? maxs : 1;
    if (one_tile) split = 1;
  }
  if (split > g.groups) split = (int)g.groups;  // no empty K ranges
  if (moe || P.layer.otype == QDG_O_I32) split = 1;  // raw integer results are not split
  ch.sc.split = split;
  ch.partial_bytes = split > 1 ? (size_t)nblocks * ch.grid_m * split * ch.sc.mt * nt * 4 * 64 * 4 : 0;
  return ch;
}

int auto_range(int64_t M) {
  int b = 0;
  while (b < kAutoRanges - 1 && ((int64_t)1 << b) < M) ++b;
  return b;
}

// The instance serving M rows: a user tuning, else an autotuned entry for
// M's range, else the device heuristics.
Choice choose(const qdg_plan& P, int64_t M) {
  if (!P.has_tuning) {
    const AutoEntry& e = P.autot[auto_range(M)];
    if (e.valid) {
      Choice c = choose_t(P, M, e.tuning, true);
      c.autotuned = true;
      return c;
    }
  }
  return choose_t(P, M, P.tuning, P.has_tuning);
}

bool instance_exists(Format f, const Choice& c) {
  return c.qtile ? true : c.tile ? tile_cfg_supported(f, c.tc) : c.ws || stream_cfg_supported(f, c.sc);
}

// Checks a tuning against the implemented kernel instances (shapes only;
// whether an instance exists for the resulting choice is checked apart).
qdg_status check_tuning(const qdg_layer_config& layer, const qdg_compute_config& compute, Format f,
                        const qdg_tuning_config& tuning) {
  const bool dense_tiled = compute.kind == QDG_KIND_DENSE && !compute.batch_invariant;
  const bool tile_ok = dense_tiled && (tuning.block_m == 128 || (f == FMT_W4A16 && tuning.block_m == 256));
  // dense W4A16: block_m 64 with block_n 512 names the 64 x 512 tiles
  const bool tile64 = dense_tiled && f == FMT_W4A16 && tuning.block_m == 64 && tuning.block_n == 512;
  // grouped MoE W4A16: block_n 512 asks for 16 x 512 tiles for 16-row blocks
  const bool moe_tile16 = compute.kind == QDG_KIND_MOE && !compute.batch_invariant && f == FMT_W4A16 &&
                          tuning.block_n == 512 && (!tuning.block_m || tuning.block_m == 16);
  if (moe_tile16) {
    if (tuning.waves && tuning.waves != 8) return fail(QDG_ERR_UNSUPPORTED, "16 x 512 tiles run 8 waves");
    if (tuning.block_k && tuning.block_k != 128) return fail(QDG_ERR_UNSUPPORTED, "block_k must be 128");
    if (tuning.mfma && tuning.mfma != 16) return fail(QDG_ERR_UNSUPPORTED, "mfma must be 16 (16x16 tiles)");
    if (tuning.split_k > 1) return fail(QDG_ERR_UNSUPPORTED, "grouped MoE does not split K");
    return QDG_OK;
  }
  if (tile64) {
    if (tuning.waves && tuning.waves != 8) return fail(QDG_ERR_UNSUPPORTED, "64 x 512 tiles run 8 waves");
    if (tuning.block_k && tuning.block_k != 128) return fail(QDG_ERR_UNSUPPORTED, "block_k must be 128");
    if (tuning.mfma && tuning.mfma != 16) return fail(QDG_ERR_UNSUPPORTED, "mfma must be 16 (16x16 tiles)");
    if (tuning.split_k < 0) return fail(QDG_ERR_INVALID_ARG, "split_k < 0");
    return QDG_OK;
  }
  if (tuning.block_m && tuning.block_m != 16 && tuning.block_m != 32 && tuning.block_m != 64 && !tile_ok)
    return fail(QDG_ERR_UNSUPPORTED,
                "block_m %d: implemented 16, 32, 64 (dense: 128; dense W4A16: 256)", tuning.block_m);
  if (tuning.block_m >= 128) {
    if (tuning.block_n && tuning.block_n != (tuning.block_m == 256 ? 128 : 256))
      return fail(QDG_ERR_UNSUPPORTED, "the tiled families pair block_m 256 with block_n 128, 128 with 256");
    if (f != FMT_W4A16 && tuning.waves && tuning.waves != 8)
      return fail(QDG_ERR_UNSUPPORTED, "the 8-bit-activation tiled family runs 8 waves");
    if (f != FMT_W4A16 && layer.otype == QDG_O_I32 && tuning.split_k > 1)
      return fail(QDG_ERR_UNSUPPORTED, "raw int32 output is not split");
  } else if (tuning.block_n && (tuning.block_n % 16 || tuning.block_n > 64)) {
    return fail(QDG_ERR_UNSUPPORTED, "block_n %d: implemented 16, 32, 64", tuning.block_n);
  }
  if (tuning.block_k && tuning.block_k != 128) return fail(QDG_ERR_UNSUPPORTED, "block_k must be 128");
  if (tuning.waves && tuning.waves != 4 && tuning.waves != 8)
    return fail(QDG_ERR_UNSUPPORTED, "waves must be 4 (streaming, tiled) or 8 (weight streaming, tiled)");
  if (tuning.mfma && tuning.mfma != 16) return fail(QDG_ERR_UNSUPPORTED, "mfma must be 16 (16x16 tiles)");
  if (tuning.split_k < 0) return fail(QDG_ERR_INVALID_ARG, "split_k < 0");
  if (compute.kind == QDG_KIND_MOE && tuning.split_k > 1)
    return fail(QDG_ERR_UNSUPPORTED, "grouped MoE does not split K");
  return QDG_OK;
}

}  // namespace

static qdg_status choose_moe(const qdg_plan& plan, int64_t T, int32_t block_m, int32_t a_per_pair, Choice* out);

extern "C" {

const char* qdg_version(void) { return "qdg 0.1.0 gfx950 layout 1"; }

const char* qdg_last_error(void) { return g_last_error.c_str(); }

qdg_status qdg_validate_layer(const qdg_layer_config* layer) { return validate_layer(layer); }

qdg_status qdg_preprocess_query(const qdg_layer_config* layer, size_t* packed_bytes) {
  qdg_status st = validate_layer(layer);
  if (st != QDG_OK) return st;
  if (!packed_bytes) return fail(QDG_ERR_INVALID_ARG, "packed_bytes is NULL");
  const PackedGeom g = packed_geom(*layer, format_of(*layer));
  *packed_bytes = (size_t)(g.expert_stride * g.experts);
  return ok();
}

qdg_status qdg_preprocess(const qdg_layer_config* layer, const qdg_std_weights* w, void* packed,
                          size_t packed_bytes, uint32_t* status, void* stream) {
  qdg_status st = validate_layer(layer);
  if (st != QDG_OK) return st;
  if (!w || !w->qweight || !w->scales || !packed) return fail(QDG_ERR_INVALID_ARG, "NULL weight or packed pointer");
  if ((layer->wtype == QDG_W_UINT4 || layer->wtype == QDG_W_UINT2) && !w->zeros)
    return fail(QDG_ERR_INVALID_ARG, "UINT4 / UINT2 weights need zero points");
  if (layer->wtype == QDG_W_NVFP4 && (!w->tensor_scale || !aligned(w->tensor_scale, 4)))
    return fail(QDG_ERR_INVALID_ARG, "NVFP4 weights need 4-byte aligned per-tensor scales");
  const Format f = format_of(*layer);
  const PackedGeom g = packed_geom(*layer, f);
  if (packed_bytes < (size_t)(g.expert_stride * g.experts))
    return fail(QDG_ERR_INVALID_ARG, "packed buffer has %zu bytes, needs %lld", packed_bytes,
                (long long)(g.expert_stride * g.experts));
  if (!aligned(packed, 256)) return fail(QDG_ERR_MISALIGNED, "packed buffer must be 256-byte aligned");
  if (!aligned(w->qweight, 16)) return fail(QDG_ERR_MISALIGNED, "qweight must be 16-byte aligned");
  if (!aligned(w->scales, 4)) return fail(QDG_ERR_MISALIGNED, "scales must be 4-byte aligned");
  if (!aligned(status, 4)) return fail(QDG_ERR_MISALIGNED, "status must be 4-byte aligned");
  return hip_status(launch_preprocess(*layer, f, g, *w, packed, status, (hipStream_t)stream), "preprocess launch");
}

qdg_status qdg_quantize_weights(const qdg_layer_config* layer, const float* w, void* qweight, void* scales,
                                void* zeros, void* stream) {
  qdg_status st = validate_layer(layer);
  if (st != QDG_OK) return st;
  if (!w || !qweight || !scales) return fail(QDG_ERR_INVALID_ARG, "NULL pointer");
  if ((layer->wtype == QDG_W_UINT4 || layer->wtype == QDG_W_UINT2) && !zeros)
    return fail(QDG_ERR_INVALID_ARG, "UINT4 / UINT2 need a zeros buffer");
  if (layer->wtype == QDG_W_NVFP4 && (!zeros || !aligned(zeros, 4)))
    return fail(QDG_ERR_INVALID_ARG, "NVFP4 needs a 4-byte aligned f32 [E] buffer for the tensor scales (zeros)");
  return hip_status(launch_quantize_weights(*layer, w, qweight, scales, zeros, (hipStream_t)stream),
                    "quantize_weights launch");
}

qdg_status qdg_quantize_act(const qdg_layer_config* layer, const void* a, int64_t M, void* qa, float* scales,
                            void* stream) {
  qdg_status st = validate_layer(layer);
  if (st != QDG_OK) return st;
  if (layer->atype != QDG_A_INT8 && layer->atype != QDG_A_FP8E4M3 && layer->atype != QDG_A_MXFP4)
    return fail(QDG_ERR_UNSUPPORTED, "this layer takes bf16 activations directly");
  if (M < 0) return fail(QDG_ERR_INVALID_ARG, "M < 0");
  if (M == 0) return ok();
  if (M > 0x7FFFFFFF) return fail(QDG_ERR_UNSUPPORTED, "M too large");
  if (!a || !qa || !scales) return fail(QDG_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned(a, 16) || !aligned(qa, 16) || !aligned(scales, 4))
    return fail(QDG_ERR_MISALIGNED, "activations must be 16-byte aligned");
  return hip_status(launch_quantize_act(layer->atype, a, M, layer->k, qa, scales, (hipStream_t)stream),
                    "quantize_act launch");
}

qdg_status qdg_plan_create(const qdg_layer_config* layer, const qdg_compute_config* compute,
                           const qdg_tuning_config* tuning, qdg_plan** out) {
  qdg_status st = validate_layer(layer);
  if (st != QDG_OK) return st;
  if (!compute || !out) return fail(QDG_ERR_INVALID_ARG, "NULL compute config or output");
  if (compute->kind != QDG_KIND_DENSE && compute->kind != QDG_KIND_MOE)
    return fail(QDG_ERR_INVALID_ARG, "bad kind %d", compute->kind);
  const Format f = format_of(*layer);
  if (compute->kind == QDG_KIND_MOE) {
    if (f == FMT_W4A16 && layer->wtype != QDG_W_INT4)
      return fail(QDG_ERR_UNSUPPORTED, "grouped W4A16 MoE is implemented for int4 symmetric weights only");
    if (compute->top_k < 1 || compute->top_k > 32) return fail(QDG_ERR_INVALID_ARG, "top_k must be in [1, 32]");
  } else if (layer->num_experts != 1) {
    return fail(QDG_ERR_INVALID_ARG, "a dense layer has num_experts = 1");
  }
  if (compute->epilogue != QDG_EPI_NONE) {
    if (compute->epilogue != QDG_EPI_SILU_MUL) return fail(QDG_ERR_INVALID_ARG, "bad epilogue %d", compute->epilogue);
    if (compute->kind != QDG_KIND_MOE)
      return fail(QDG_ERR_UNSUPPORTED, "the SiLU*mul epilogue is implemented for MoE plans");
    if (layer->n % 32 != 0)
      return fail(QDG_ERR_UNSUPPORTED, "SiLU*mul needs n = 2*I with I a multiple of 16 (n=%lld)", (long long)layer->n);
    if (layer->otype == QDG_O_I32) return fail(QDG_ERR_UNSUPPORTED, "SiLU*mul has no int32 output");
  }
  if (tuning) {
    st = check_tuning(*layer, *compute, f, *tuning);
    if (st != QDG_OK) return st;
  }
  qdg_plan* p = new (std::nothrow) qdg_plan;
  if (!p) return fail(QDG_ERR_INVALID_ARG, "out of host memory");
  std::memset(p->autot, 0, sizeof p->autot);
  p->layer = *layer;
  p->compute = *compute;
  p->has_tuning = tuning != nullptr;
  if (tuning) p->tuning = *tuning;
  else std::memset(&p->tuning, 0, sizeof p->tuning);
  p->fmt = f;
  p->geom = packed_geom(*layer, f);
  if (tuning) {
    // grouped plans: the instance of one token in blocks of the tuning's
    // block_m (16 when it names none)
    Choice c;
    bool exists;
    if (compute->kind == QDG_KIND_MOE) {
      const int bm = tuning->block_m ? tuning->block_m : 16;
      exists = choose_moe(*p, 1, bm, 0, &c) == QDG_OK && instance_exists(f, c);
    } else {
      c = choose(*p, 1);
      exists = instance_exists(f, c);
    }
    if (!exists) {
      delete p;
      return fail(QDG_ERR_UNSUPPORTED, "no kernel instance for block_m/block_n/waves of this tuning");
    }
  }
  *out = p;
  return ok();
}

void qdg_plan_destroy(qdg_plan* plan) { delete plan; }

qdg_status qdg_plan_workspace(const qdg_plan* plan, int64_t M, size_t* bytes) {
  if (!plan || !bytes) return fail(QDG_ERR_INVALID_ARG, "NULL plan or output");
  if (M < 0) return fail(QDG_ERR_INVALID_ARG, "M < 0");
  const Choice c = choose(*plan, M > 0 ? M : 1);
  int64_t rowsum = (int64_t)c.rowsum_bytes;
  if (plan->compute.kind == QDG_KIND_MOE &&
      (plan->fmt == FMT_W4A16 || plan->fmt == FMT_W8A16 || plan->fmt == FMT_W2A16)) {
    // MoE: room for the row sums of 128-row blocks (the largest block size)
    const int64_t cap =
        align_up((M > 0 ? M : 1) * plan->compute.top_k + plan->layer.num_experts * 127, 128);
    rowsum = cap * plan->geom.groups * 4;
  }
  if (plan->fmt == FMT_MXFP4_I8) {
    // the two E4M3 planes of the int8 activations (MoE: room for one row per
    // (token, slot), the per-pair input of a down projection)
    const int64_t rows = (M > 0 ? M : 1) * (plan->compute.kind == QDG_KIND_MOE ? plan->compute.top_k : 1);
    rowsum = 2 * rows * plan->layer.k;
  }
  *bytes = kCounterBytes + align_up((int64_t)c.partial_bytes, 256) + align_up(rowsum, 256);
  return ok();
}

// Kernel choice of a grouped MoE call: the caller's block size decides the
// family. W4A16: 16-row blocks run the streaming family (the LDS-tiled one
// when K is short, weight streaming when a tuning pins it), 32-, 64- and
// 128-row blocks the LDS-tiled family; the other formats as noted below.
static qdg_status choose_moe(const qdg_plan& plan, int64_t T, int32_t block_m, int32_t a_per_pair, Choice* out) {
  const Choice c0 = choose(plan, T);
  Choice c = c0;
  const int64_t rows = T * plan.compute.top_k;
  c.sc.mt = block_m / 16;
  c.sc.split = 1;
  c.partial_bytes = 0;
  const int64_t E = plan.layer.num_experts;
  const int64_t cap = align_up(rows + E * (block_m - 1), block_m);
  c.grid_m = (int)(cap / block_m);
  const qdg_tuning_config& tu = plan.tuning;
  // 16-row blocks: the streaming family with four 16-column tiles per wave
  // (measured on MI355X at E = 256, hidden 7168: 29 % faster than weight
  // streaming for gate+up at T = 64, a few % for down and at T = 512, since
  // each expert block would otherwise restage its A rows per workgroup),
  // unless a tuning pins weight streaming
  const bool ws_pinned = plan.has_tuning && tu.block_n == 64 && tu.waves == 8;
  const bool silu = plan.compute.epilogue == QDG_EPI_SILU_MUL;  // weight streaming has no such epilogue
  c.ws = block_m == 16 && !plan.compute.batch_invariant && !silu && ws_pinned;
  if (plan.fmt != FMT_W4A16) {
    // every other format: the streaming family, block_m / 16 row tiles; 128-row
    // blocks (plain output only) run in the LDS-tiled families: NVFP4, W8A16
    // and W2A16 in the bf16 one, W8A8, W4A8 and the MXFP4 formats in the
    // 8-bit one
    const bool tiled_fmt = plan.fmt == FMT_NVFP4 || plan.fmt == FMT_W8A16 || plan.fmt == FMT_W2A16;
    const bool qtiled_fmt = plan.fmt == FMT_W8A8 || plan.fmt == FMT_W4A8 || plan.fmt == FMT_MXFP4 ||
                            plan.fmt == FMT_W4A4 || plan.fmt == FMT_MXFP4_I8;
    const bool tiled = (block_m == 128 || (block_m == 64 && qtiled_fmt)) && (tiled_fmt || qtiled_fmt) && !silu &&
                       !plan.compute.batch_invariant;
    if (block_m > 64 && !tiled)
      return fail(QDG_ERR_UNSUPPORTED, "grouped MoE of %s uses block_m 16, 32 or 64%s", fmt_name(plan.fmt, plan.layer),
                  tiled_fmt || qtiled_fmt ? " (128 without an epilogue)" : "");
    c.ws = c.tile = c.qtile = false;
    c.sc = StreamCfg{block_m / 16, 2, 4, 1};
    c.rowsum_bytes = 0;
    if (tiled) {
      // A rows are addressed with 32-bit byte offsets in the tiled families
      const int64_t a_rows = a_per_pair ? rows : T;
      const double a_row_bytes = tiled_fmt || plan.fmt == FMT_MXFP4_I8 ? 2.0 * plan.layer.k
                                 : plan.fmt == FMT_W4A4             ? plan.layer.k / 2.0
                                                                    : (double)plan.layer.k;
      if ((double)a_rows * a_row_bytes >= 4294967296.0)
        return fail(QDG_ERR_UNSUPPORTED, "A of %lld rows is too large for 128-row MoE blocks", (long long)a_rows);
      c.tc = block_m == 64 ? TileCfg{64, 512, 8} : TileCfg{128, 256, 8};
      if (tiled_fmt) {
        c.tile = true;
        if (plan.fmt != FMT_NVFP4) c.rowsum_bytes = (size_t)c.grid_m * 128 * plan.geom.groups * 4;
      } else {
        c.qtile = true;
        // while experts hold at most one block of rows on average, most
        // blocks are partly filled and the instance that skips their
        // all-padding 32-row halves wins (measured on MI355X, W4A8-INT8 at
        // E = 256, top-8, hidden 7168, 64-row blocks: T = 512 gate+up
        // 828-846 -> 773-782 us, down 521-524 -> 481 us); with more rows it
        // loses (T = 4096: 1932-1944 -> 2027-2041 us)
        c.pad_skip = rows <= E * block_m;
      }
    }
    *out = c;
    return QDG_OK;
  }
  if (c.ws) c.sc = StreamCfg{1, 4, 8, 1};  // 16 x 64 per workgroup of 8 waves
  else if (!plan.has_tuning || c0.tile || c0.ws || !stream_cfg_supported(plan.fmt, c.sc))
    c.sc = StreamCfg{block_m / 16, block_m == 16 ? 4 : 2, 4, 1};
  c.tile = false;
  c.qtile = false;
  // 32-, 64- and 128-row blocks: the LDS-tiled family (32 x 512, 64 x 512
  // and 128 x 256 tiles). Measured on MI355X at E = 256, hidden 7168: at
  // T = 512 32-row blocks in it run gate+up in 842 us and down in 449 us,
  // against 1259 and 758 us for 16-row streaming blocks; at T = 4096 64-row
  // blocks run gate+up in 2842 us and down in 1583 us against 3203 and
  // 1813 us with 128-row blocks (less padding per expert), where 64-row
  // streaming blocks took 7.1 and 7.4 ms
  // 16-row blocks: 16 x 512 tiles of the LDS-tiled family when a tuning asks
  // for them (block_n 512) or, without a tuning, when K holds at most 16
  // groups. Measured on MI355X at E = 256, T = 64: the down projection
  // (K = 2048, N = 7168) in 321 us against 380 us in the streaming family
  // (whose workgroups then hold 4 groups per wave), gate+up (K = 7168) in
  // 609 against 587 us
  const bool tile16 = block_m == 16 && !plan.compute.batch_invariant && !c.ws &&
                      (plan.has_tuning ? tu.block_n == 512 : plan.geom.groups <= 16);
  if (block_m == 128 || tile16 || ((block_m == 32 || block_m == 64) && !plan.compute.batch_invariant)) {
    // A rows are addressed with 32-bit byte offsets in the tiled family
    const int64_t a_rows = a_per_pair ? rows : T;
    if ((double)a_rows * (double)plan.layer.k * 2.0 >= 4294967296.0)
      return fail(QDG_ERR_UNSUPPORTED, "A of %lld rows is too large for %d-row MoE blocks", (long long)a_rows,
                  block_m);
    if (plan.compute.batch_invariant)
      return fail(QDG_ERR_UNSUPPORTED, "batch-invariant MoE plans use block_m <= 64");
    c.tile = true;
    c.ws = false;
    c.tc = block_m == 128 ? TileCfg{128, 256, 8} : TileCfg{block_m, 512, 8};
  } else if (!c.ws && !stream_cfg_supported(plan.fmt, c.sc)) {
    return fail(QDG_ERR_UNSUPPORTED, "block_m %d unsupported", block_m);
  }
  if (silu && !c.tile && c.sc.nt != 2 && c.sc.nt != 4)
    return fail(QDG_ERR_UNSUPPORTED, "the SiLU*mul epilogue pairs gate and up tiles: block_n must be 32 or 64");
  *out = c;
  return QDG_OK;
}

// The MFMA instruction an instance issues.
static const char* mfma_name(Format f, const Choice& c) {
  if (f == FMT_W4A16) return c.tile && c.tc.bm * c.tc.bn / (64 * c.tc.waves) == 64 ? "32x32x16_bf16" : "16x16x32_bf16";
  if (f == FMT_W8A16 || f == FMT_NVFP4) return c.tile ? "32x32x16_bf16" : "16x16x32_bf16";
  if (f == FMT_W2A16) return c.tile ? "32x32x16_bf16" : "16x16x32_bf16";
  if (f == FMT_MXFP4) return "scale_16x16x128_f8f6f4";
  if (f == FMT_W4A4) return "scale_16x16x128_f4f4";
  if (f == FMT_MXFP4_I8) return "2x_scale_16x16x128_f8f6f4";
  return "16x16x64_i8";
}

// The main kernel of a weight-streaming, LDS-tiled or 8-bit LDS-tiled
// choice: launched, or (desc set) described without launching anything.
static hipError_t family_launch(const qdg_plan& plan, const Choice& c, const GemmArgs& a, bool moe, hipStream_t s,
                                KernelLaunch* desc) {
  const bool asym = plan.layer.wtype == QDG_W_UINT4;
  if (c.qtile) return launch_qtile(plan.fmt, moe, c.tc.bm, c.pad_skip, a, c.grid_m, s, desc);
  if (c.tile) return launch_tile(plan.fmt, asym, moe, c.tc, a, c.grid_m, s, desc);
  return plan.fmt == FMT_W4A16 ? launch_wstream(asym, moe, a, c.sc.split, c.grid_m, s, desc)
                               : launch_wstream8(plan.fmt, a, c.sc.split, c.sc.nt, s, desc);
}

static const JitInstance* find_jit_expr(const qdg_plan& plan, const char* expr, bool moe) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  for (const JitInstance& j : plan.jit)
    if (!j.expr.empty() && j.expr == expr && j.moe == moe && j.device == dev) return &j;
  return nullptr;
}

// The size fields a launcher reads to pick its kernel and grid.
static GemmArgs shape_args(const qdg_plan& plan, const Choice& c) {
  GemmArgs a{};
  a.N = (int)plan.layer.n;
  a.K = (int)plan.layer.k;
  a.groups = (int)plan.geom.groups;
  a.ntiles = (int)plan.geom.ntiles;
  a.otype = plan.layer.otype;
  a.split = c.sc.split;
  a.epi = plan.compute.epilogue;
  return a;
}

static const JitInstance* find_jit(const qdg_plan& plan, const Choice& c, bool moe) {
  if (plan.jit.empty()) return nullptr;
  if (c.ws || c.tile || c.qtile) {
    KernelLaunch d{};
    if (family_launch(plan, c, shape_args(plan, c), moe, nullptr, &d) != hipSuccess) return nullptr;
    return find_jit_expr(plan, d.expr, moe);
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  for (const JitInstance& j : plan.jit)
    if (j.expr.empty() && j.mt == c.sc.mt && j.nt == c.sc.nt && j.kw == c.sc.kw && j.moe == moe && j.device == dev)
      return &j;
  return nullptr;
}

// The main kernel of a non-streaming choice from the plan's run-time
// compiled instance when it has one (the weight-streaming split reduce
// then follows here), else ahead of time.
static hipError_t launch_main(const qdg_plan& plan, const Choice& c, const GemmArgs& a, bool moe, hipStream_t s) {
  if (!plan.jit.empty()) {
    KernelLaunch d{};
    if (family_launch(plan, c, a, moe, s, &d) == hipSuccess) {
      if (const JitInstance* j = find_jit_expr(plan, d.expr, moe)) {
        hipError_t e = launch_jit(j->fn, d, a, s);
        if (e == hipSuccess && c.ws && !moe && c.sc.split > 1) e = launch_reduce_splits(a, 16, a.ntiles * 16, s);
        return e;
      }
    }
  }
  return family_launch(plan, c, a, moe, s, nullptr);
}

static int describe(const qdg_plan& plan, const Choice& c, int64_t M, const char* kind, char* buf, size_t len) {
  return snprintf(buf, buf ? len : 0,
                  "%s %s n=%lld k=%lld E=%lld M=%lld: family=%s block_m=%d block_n=%d split_k=%d "
                  "waves=%d mfma=%s grid_m=%d batch_invariant=%d epilogue=%s%s tuning=%s code=%s layout=%d arch=gfx950",
                  fmt_name(plan.fmt, plan.layer), kind, (long long)plan.layer.n, (long long)plan.layer.k,
                  (long long)plan.layer.num_experts, (long long)M,
                  c.qtile ? "qtile" : c.tile ? "tile" : c.ws ? "wstream" : "stream",
                  c.tile || c.qtile ? c.tc.bm : c.sc.mt * 16, c.tile || c.qtile ? c.tc.bn : c.sc.nt * 16,
                  c.sc.split, c.tile || c.qtile ? c.tc.waves : c.sc.kw, mfma_name(plan.fmt, c), c.grid_m,
                  plan.compute.batch_invariant, plan.compute.epilogue == QDG_EPI_SILU_MUL ? "silu_mul" : "none",
                  c.pad_skip ? " pad_skip=1" : "", c.autotuned ? "autotuned" : plan.has_tuning ? "user" : "heuristic",
                  find_jit(plan, c, plan.compute.kind == QDG_KIND_MOE) ? "jit" : "aot", QDG_LAYOUT_VERSION);
}

int qdg_plan_describe(const qdg_plan* plan, int64_t M, char* buf, size_t len) {
  if (!plan || M < 0) return -1;
  const Choice c = choose(*plan, M > 0 ? M : 1);
  return describe(*plan, c, M, plan->compute.kind == QDG_KIND_MOE ? "moe" : "dense", buf, len);
}

int qdg_moe_describe(const qdg_plan* plan, int64_t T, int32_t block_m, char* buf, size_t len) {
  if (!plan || T < 0 || plan->compute.kind != QDG_KIND_MOE) return -1;
  if (block_m != 16 && block_m != 32 && block_m != 64 && block_m != 128) return -1;
  Choice c;
  if (choose_moe(*plan, T > 0 ? T : 1, block_m, 0, &c) != QDG_OK) return -1;
  return describe(*plan, c, T, "moe", buf, len);
}

static qdg_status run(const qdg_plan* plan, const void* A, const float* a_scales, const void* packed, void* Y,
                      int64_t M, void* workspace, size_t ws_bytes, hipStream_t stream, bool moe,
                      const int32_t* sorted_ids, const int32_t* block_expert, const int32_t* num_padded,
                      int64_t T, int32_t block_m, int32_t a_per_pair) {
  Choice c = choose(*plan, M);
  int64_t rows = M;
  if (moe) {
    rows = T * plan->compute.top_k;
    const qdg_status st = choose_moe(*plan, T, block_m, a_per_pair, &c);
    if (st != QDG_OK) return st;
  }
  size_t need = 0;
  qdg_plan_workspace(plan, M, &need);
  if (!workspace || ws_bytes < need)
    return fail(QDG_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws_bytes, need);
  if (!aligned(workspace, 256)) return fail(QDG_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  GemmArgs a{};
  a.A = A;
  a.a_scales = a_scales;
  a.packed = (const uint8_t*)packed;
  a.Y = Y;
  a.M = (int)M;
  a.N = (int)plan->layer.n;
  a.K = (int)plan->layer.k;
  a.groups = (int)plan->geom.groups;
  a.ntiles = (int)plan->geom.ntiles;
  a.expert_stride = plan->geom.expert_stride;
  a.s_offset = plan->geom.s_offset;
  a.otype = plan->layer.otype;
  a.split = c.sc.split;
  a.counters = (unsigned*)workspace;
  a.partial = (char*)workspace + kCounterBytes;
  a.sorted_ids = sorted_ids;
  a.block_expert = block_expert;
  a.num_padded = num_padded;
  a.top_k = plan->compute.top_k;
  a.a_per_pair = a_per_pair;
  a.num_pairs = (int)rows;
  a.epi = plan->compute.epilogue;
  a.unpack_mask = plan->fmt == FMT_W2A16 ? 0x00030003u : 0x000F000Fu;
  a.unpack_exp = 0x43004300u;
  const bool asym = plan->layer.wtype == QDG_W_UINT4;
  hipError_t e;
  if (plan->fmt == FMT_MXFP4_I8) {
    // the int8 codes become two E4M3 planes in the workspace (either family)
    const int64_t a_rows = moe ? (a_per_pair ? rows : T) : M;
    uint8_t* pl = (uint8_t*)workspace + kCounterBytes + align_up((int64_t)c.partial_bytes, 256);
    e = launch_act_i8_planes((const int8_t*)A, a_rows, a.K, pl, stream);
    if (e != hipSuccess) return hip_status(e, "activation planes launch");
    a.A = pl;
  }
  if (c.qtile) {
    a.m_pad = c.grid_m * c.tc.bm;
    e = launch_main(*plan, c, a, moe, stream);
    if (e == hipSuccess && a.split > 1) {
      const int n_pad = (int)((plan->geom.ntiles + 15) / 16 * 256);
      e = launch_reduce_splits(a, a.m_pad, n_pad, stream);
    }
  } else if (c.tile) {
    a.m_pad = c.grid_m * c.tc.bm;
    float* rs = (float*)((char*)workspace + kCounterBytes + align_up((int64_t)c.partial_bytes, 256));
    a.rowsum = rs;
    // offsets: -(128 + z) per group for UINT4 (applied in the kernel), 136 for
    // INT4 and 128 for INT8 (pre-scaled here)
    const float rs_factor = plan->fmt == FMT_W8A16 ? -128.0f : asym || plan->fmt == FMT_W2A16 ? 1.0f : -136.0f;
    if (plan->fmt == FMT_NVFP4)  // scaled weights: no row-sum offsets
      e = hipSuccess;
    else
      e = moe ? launch_rowsum(A, sorted_ids, num_padded, a.top_k, a_per_pair, (int)rows, (int)M, a.K, a.m_pad,
                              rs_factor, rs, stream)
              : launch_rowsum(A, nullptr, nullptr, 0, 0, (int)rows, (int)M, a.K, a.m_pad, rs_factor, rs,
                              stream);
    if (e != hipSuccess) return hip_status(e, "rowsum launch");
    e = launch_main(*plan, c, a, moe, stream);
    if (e == hipSuccess && a.split > 1) {
      const int n_pad = (int)((plan->geom.ntiles + c.tc.bn / 16 - 1) / (c.tc.bn / 16) * c.tc.bn);
      e = launch_reduce_splits(a, a.m_pad, n_pad, stream);
    }
  } else if (c.ws) {
    e = launch_main(*plan, c, a, moe, stream);
  } else {
    // the streaming family addresses A with 31-bit byte offsets
    const int64_t a_rows = moe ? (a_per_pair ? rows : T) : M;
    const bool bf16_a = plan->fmt == FMT_W4A16 || plan->fmt == FMT_W8A16 || plan->fmt == FMT_NVFP4 ||
                        plan->fmt == FMT_W2A16;
    const bool planes = plan->fmt == FMT_MXFP4_I8;  // int8 codes become two E4M3 planes
    a.a_bytes = a_rows * (bf16_a || planes ? 2 * (int64_t)a.K : plan->fmt == FMT_W4A4 ? a.K / 2 : a.K);
    if (a.a_bytes >= ((int64_t)1 << 31))
      return fail(QDG_ERR_UNSUPPORTED, "A of %lld bytes is too large for the streaming family (< 2 GiB)",
                  (long long)a.a_bytes);
    a.m_pad = c.grid_m * c.sc.mt * 16;
    const JitInstance* jit = find_jit(*plan, c, moe);
    e = jit ? launch_stream_jit(jit->fn, c.sc, a, c.grid_m, stream)
            : launch_stream(plan->fmt, asym, moe, c.sc, a, c.grid_m, stream);
    if (e == hipSuccess && a.split > 1) {
      const int n_pad = (int)((plan->geom.ntiles + c.sc.nt - 1) / c.sc.nt * c.sc.nt * 16);
      e = launch_reduce_splits(a, a.m_pad, n_pad, stream);
    }
  }
  if (e == hipErrorInvalidValue) return fail(QDG_ERR_UNSUPPORTED, "no kernel instance for this tuning");
  return hip_status(e, "gemm launch");
}

qdg_status qdg_gemm(const qdg_plan* plan, const void* A, const float* a_scales, const void* packed, void* Y,
                    int64_t M, void* workspace, size_t ws_bytes, void* stream) {
  if (!plan) return fail(QDG_ERR_INVALID_ARG, "plan is NULL");
  if (plan->compute.kind != QDG_KIND_DENSE) return fail(QDG_ERR_INVALID_ARG, "MoE plans run with qdg_moe_gemm");
  if (M < 0) return fail(QDG_ERR_INVALID_ARG, "M < 0");
  if (M == 0) return ok();
  if (M > 0x7FFFFFFF / 2) return fail(QDG_ERR_UNSUPPORTED, "M too large");
  if (!A || !packed || !Y) return fail(QDG_ERR_INVALID_ARG, "NULL A, packed or Y");
  const bool need_scales = plan->fmt != FMT_W4A16 && plan->fmt != FMT_W8A16 && plan->fmt != FMT_NVFP4 &&
                           plan->fmt != FMT_W2A16 &&
                           plan->layer.otype != QDG_O_I32;
  if (plan->fmt == FMT_MXFP4 || plan->fmt == FMT_W4A4 || plan->fmt == FMT_MXFP4_I8) {
    if (!a_scales) return fail(QDG_ERR_INVALID_ARG, "MXFP4 needs activation scales");
  } else if (need_scales && !a_scales) {
    return fail(QDG_ERR_INVALID_ARG, "activation scales are NULL");
  }
  if (!aligned(A, 16)) return fail(QDG_ERR_MISALIGNED, "A must be 16-byte aligned");
  if (!aligned(packed, 256)) return fail(QDG_ERR_MISALIGNED, "packed must be 256-byte aligned");
  const size_t ybytes = plan->layer.otype == QDG_O_BF16 ? 2 : 4;
  if (!aligned(Y, ybytes)) return fail(QDG_ERR_MISALIGNED, "Y must be aligned to its element size");
  return run(plan, A, a_scales, packed, Y, M, workspace, ws_bytes, (hipStream_t)stream, false, nullptr, nullptr,
             nullptr, 0, 0, 0);
}

// Candidate tunings for M rows: every kernel family that can serve M, with
// its tile shapes and (weight streaming) K splits; split 0 keeps the family's
// split heuristic. Candidates without an instance are dropped by the caller.
static void autotune_candidates(const qdg_plan& P, int64_t M, qdg_tuning_config* out, int* n, int cap) {
  *n = 0;
  auto add = [&](int bm, int bn, int split, int waves) {
    if (*n >= cap) return;
    qdg_tuning_config t;
    std::memset(&t, 0, sizeof t);
    t.block_m = bm;
    t.block_n = bn;
    t.split_k = split;
    t.waves = waves;
    out[(*n)++] = t;
  };
  if (M <= 16) {  // weight streaming
    if (P.fmt == FMT_W4A16) {
      for (int s : {0, 1, 2, 4, 8}) add(16, 64, s, 8);
    } else {
      add(16, 64, 0, 8);
    }
  }
  if (M <= 256) {  // streaming: the smallest row block that holds M, and larger ones
    for (int bm = M <= 16 ? 16 : M <= 32 ? 32 : 64; bm <= 64; bm *= 2)
      for (int bn : {16, 32, 64}) add(bm, bn, 0, 4);
    if (M <= 64)
      for (int bn : {16, 32, 64}) add(M <= 16 ? 16 : M <= 32 ? 32 : 64, bn, 1, 4);  // unsplit
  }
  if (M > 16) {  // LDS-tiled, with the K-split heuristic and fixed splits
    for (int s : {0, 1, 2, 4, 8}) add(128, 256, s, 8);
    if (P.fmt == FMT_W4A16) {
      add(128, 256, 0, 4);
      if (M > 128) add(256, 128, 0, 8);
      if (M <= 128)
        for (int s : {0, 2, 4, 8}) add(64, 512, s, 8);
    }
  }
}

// Two choices launch the same kernel instance on the same grid.
static bool same_instance(const Choice& a, const Choice& b) {
  if (a.tile != b.tile || a.ws != b.ws || a.qtile != b.qtile || a.grid_m != b.grid_m) return false;
  if (a.sc.mt != b.sc.mt || a.sc.nt != b.sc.nt || a.sc.kw != b.sc.kw || a.sc.split != b.sc.split) return false;
  return !a.tile || (a.tc.bm == b.tc.bm && a.tc.bn == b.tc.bn && a.tc.waves == b.tc.waves);
}

// A tuning under which choose_t picks the heuristic's instance for M rows
// (false if none does).
static bool tuning_of_heuristic(const qdg_plan& P, int64_t M, qdg_tuning_config* out) {
  const Choice h = choose_t(P, M, P.tuning, false);
  qdg_tuning_config t;
  std::memset(&t, 0, sizeof t);
  t.block_m = h.tile ? h.tc.bm : h.ws ? 16 : h.sc.mt * 16;
  t.block_n = h.tile ? h.tc.bn : h.ws ? 0 : h.sc.nt * 16;
  t.split_k = h.sc.split;
  t.waves = h.tile ? h.tc.waves : h.ws ? 0 : h.sc.kw;
  if (check_tuning(P.layer, P.compute, P.fmt, t) != QDG_OK) return false;
  if (!same_instance(choose_t(P, M, t, true), h)) return false;
  *out = t;
  return true;
}

// Weight copies the autotuner rotates over: together at least twice the
// 256 MB last-level cache (MALL) of MI355X, so that no timed launch finds
// its weights cache-resident from the launch before.
constexpr size_t kRotateBytes = (size_t)512 << 20;
constexpr int kMaxCopies = 64;
// A candidate replaces the heuristic's instance only when it is faster by
// more than the timing noise.
constexpr float kHeuristicMargin = 0.03f;

qdg_status qdg_plan_autotune(qdg_plan* plan, const void* A, const float* a_scales, const void* packed, void* Y,
                             int64_t M, void* workspace, size_t ws_bytes, int32_t reps, void* stream,
                             qdg_tuning_config* chosen, float* best_us) {
  if (!plan) return fail(QDG_ERR_INVALID_ARG, "plan is NULL");
  if (plan->compute.kind != QDG_KIND_DENSE) return fail(QDG_ERR_UNSUPPORTED, "autotuning is for dense plans");
  if (plan->has_tuning) return fail(QDG_ERR_UNSUPPORTED, "the plan carries a user tuning");
  if (plan->compute.batch_invariant)
    return fail(QDG_ERR_UNSUPPORTED, "a batch-invariant plan keeps one instance for every M");
  if (M < 1 || M > 0x7FFFFFFF / 2) return fail(QDG_ERR_INVALID_ARG, "M must be in [1, 2^30)");
  if (reps < 1 || reps > 1000) return fail(QDG_ERR_INVALID_ARG, "reps must be in [1, 1000]");
  if (!A || !packed || !Y || !workspace) return fail(QDG_ERR_INVALID_ARG, "NULL A, packed, Y or workspace");
  constexpr int kCap = 49;
  qdg_tuning_config cand[kCap];
  // candidate 0: the heuristic's own instance, when a tuning reproduces it
  int ncand = 0;
  const bool heur = tuning_of_heuristic(*plan, M, &cand[0]);
  if (heur) ncand = 1;
  {
    int more = 0;
    autotune_candidates(*plan, M, cand + ncand, &more, kCap - ncand);
    ncand += more;
  }
  hipStream_t st = (hipStream_t)stream;
  // weight copies to rotate over (copy 0 is the caller's buffer); without
  // device memory for them the timing uses the caller's buffer alone
  const size_t pb = align_up((int64_t)(plan->geom.expert_stride * plan->geom.experts), 256);
  int ncopies = (int)std::min<size_t>(kMaxCopies, std::max<size_t>(1, (kRotateBytes + pb - 1) / pb));
  uint8_t* rot = nullptr;
  if (ncopies > 1 && hipMalloc((void**)&rot, (ncopies - 1) * pb) != hipSuccess) {
    (void)hipGetLastError();
    rot = nullptr;
    ncopies = 1;
  }
  for (int i = 1; i < ncopies; ++i) {
    if (hipMemcpyAsync(rot + (i - 1) * pb, packed, plan->geom.expert_stride * plan->geom.experts,
                       hipMemcpyDeviceToDevice, st) != hipSuccess) {
      (void)hipFree(rot);
      return fail(QDG_ERR_HIP, "copying the weights for autotuning failed");
    }
  }
  auto copy = [&](int k) -> const void* { return k % ncopies == 0 ? packed : rot + (k % ncopies - 1) * pb; };
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    (void)hipStreamSynchronize(st);
    if (rot) (void)hipFree(rot);
    return fail(QDG_ERR_HIP, "hipEventCreate failed");
  }
  // Candidates are timed in three interleaved rounds and keep their best
  // round, so that clock ramps and drift during the sweep do not favour the
  // ones timed last.
  bool usable[kCap];
  float t_best[kCap];
  Choice inst[kCap];
  for (int i = 0; i < ncand; ++i) {
    t_best[i] = -1.f;
    usable[i] = check_tuning(plan->layer, plan->compute, plan->fmt, cand[i]) == QDG_OK;
    if (!usable[i]) continue;
    inst[i] = choose_t(*plan, M, cand[i], true);
    // candidates that launch an instance timed already are not timed again
    for (int j = 0; j < i && usable[i]; ++j)
      if (usable[j] && same_instance(inst[i], inst[j])) usable[i] = false;
  }
  qdg_status err = QDG_OK;
  for (int round = 0; round < 3 && err == QDG_OK; ++round) {
    for (int i = 0; i < ncand && err == QDG_OK; ++i) {
      if (!usable[i]) continue;
      plan->tuning = cand[i];
      plan->has_tuning = true;
      const Choice c = choose(*plan, M);
      size_t need = 0;
      usable[i] = instance_exists(plan->fmt, c) && qdg_plan_workspace(plan, M, &need) == QDG_OK && need <= ws_bytes;
      if (usable[i]) {
        // one untimed launch, then reps launches over the rotated weight
        // copies between two events
        qdg_status r = qdg_gemm(plan, A, a_scales, copy(ncopies - 1), Y, M, workspace, ws_bytes, stream);
        if (r == QDG_ERR_UNSUPPORTED || r == QDG_ERR_WORKSPACE) {
          usable[i] = false;
        } else if (r != QDG_OK) {
          err = r;
        } else {
          hipError_t h = hipEventRecord(e0, st);
          for (int k = 0; k < reps && r == QDG_OK && h == hipSuccess; ++k)
            r = qdg_gemm(plan, A, a_scales, copy(k), Y, M, workspace, ws_bytes, stream);
          if (h == hipSuccess) h = hipEventRecord(e1, st);
          if (h == hipSuccess) h = hipEventSynchronize(e1);
          float ms = 0.f;
          if (h == hipSuccess) h = hipEventElapsedTime(&ms, e0, e1);
          if (r != QDG_OK) {
            err = r;
          } else if (h != hipSuccess) {
            err = hip_status(h, "autotune timing");
          } else {
            const float us = ms * 1000.f / (float)reps;
            if (t_best[i] < 0.f || us < t_best[i]) t_best[i] = us;
          }
        }
      }
      plan->has_tuning = false;
      std::memset(&plan->tuning, 0, sizeof plan->tuning);
    }
  }
  int best = -1;
  float best_t = 0.f;
  for (int i = 0; i < ncand; ++i)
    if (usable[i] && t_best[i] >= 0.f && (best < 0 || t_best[i] < best_t)) {
      best = i;
      best_t = t_best[i];
    }
  // keep the heuristic's instance unless the winner beats it by more than noise
  if (heur && best > 0 && usable[0] && t_best[0] >= 0.f && best_t > t_best[0] * (1.f - kHeuristicMargin)) {
    best = 0;
    best_t = t_best[0];
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  (void)hipStreamSynchronize(st);  // the launches that read the copies are done
  if (rot) (void)hipFree(rot);
  if (err != QDG_OK) return err;
  if (best < 0) return fail(QDG_ERR_WORKSPACE, "no kernel instance for M = %lld fits the workspace", (long long)M);
  AutoEntry& e = plan->autot[auto_range(M)];
  e.tuning = cand[best];
  e.us = best_t;
  e.valid = true;
  if (chosen) *chosen = cand[best];
  if (best_us) *best_us = best_t;
  // leave Y holding the result of the chosen instance
  return qdg_gemm(plan, A, a_scales, packed, Y, M, workspace, ws_bytes, stream);
}

qdg_status qdg_plan_autotune_reset(qdg_plan* plan) {
  if (!plan) return fail(QDG_ERR_INVALID_ARG, "plan is NULL");
  std::memset(plan->autot, 0, sizeof plan->autot);
  return ok();
}

qdg_status qdg_plan_jit(qdg_plan* plan, int64_t M, int32_t block_m, const char* cache_dir, qdg_jit_info* info) {
  if (!plan) return fail(QDG_ERR_INVALID_ARG, "plan is NULL");
  if (M < 1) return fail(QDG_ERR_INVALID_ARG, "M must be >= 1");
  const bool moe = plan->compute.kind == QDG_KIND_MOE;
  Choice c;
  if (moe) {
    if (choose_moe(*plan, M, block_m, 0, &c) != QDG_OK) return QDG_ERR_UNSUPPORTED;
  } else {
    c = choose(*plan, M);
  }
  // Measured on MI355X: instances whose scaled MFMA multiplies fp8 (E4M3)
  // activations with fp4 weights (MXFP4, and MXFP4 x INT8 through its E4M3
  // planes) return results scaled by exactly 2^-127 when launched from the
  // hipRTC code object, in every family, although that code object is byte
  // for byte the same on every host and its instructions match the ahead-of-
  // time build; fp4 x fp4 (W4A4) and every other instance agree bit for bit.
  // Until the cause is known those two formats run ahead of time only.
  if (plan->fmt == FMT_MXFP4 || plan->fmt == FMT_MXFP4_I8)
    return fail(QDG_ERR_UNSUPPORTED, "run-time compilation of the fp8 x fp4 scaled-MFMA instances (%s) is disabled",
                fmt_name(plan->fmt, plan->layer));
  int dev = 0;
  if (c.ws || c.tile || c.qtile) {
    // the instance the plan launches for this M, described by its launcher
    KernelLaunch d{};
    if (family_launch(*plan, c, shape_args(*plan, c), moe, nullptr, &d) != hipSuccess)
      return fail(QDG_ERR_UNSUPPORTED, "no kernel instance for this M");
    JitResult r = jit_kernel(d.src, d.expr, cache_dir);
    if (!r.fn) return fail(QDG_ERR_HIP, "%s", r.error.c_str());
    (void)hipGetDevice(&dev);
    bool found = false;
    for (JitInstance& j : plan->jit)
      if (j.expr == d.expr && j.moe == moe && j.device == dev) {
        j.fn = r.fn;
        found = true;
      }
    if (!found) plan->jit.push_back(JitInstance{0, 0, 0, dev, moe, r.fn, std::string(d.expr)});
    if (info) {
      info->compile_ms = r.compile_ms;
      info->load_ms = r.load_ms;
      info->from_cache = r.from_cache;
      info->code_bytes = r.code_bytes;
      std::snprintf(info->key, sizeof info->key, "%s", r.key);
    }
    return ok();
  }
  if (!stream_cfg_supported(plan->fmt, c.sc)) return fail(QDG_ERR_UNSUPPORTED, "no streaming instance for this M");
  const bool asym = plan->layer.wtype == QDG_W_UINT4;
  const bool raw = plan->layer.otype == QDG_O_I32;
  JitResult r = jit_stream_kernel(plan->fmt, asym, raw, c.sc, moe, cache_dir);
  if (!r.fn) return fail(QDG_ERR_HIP, "%s", r.error.c_str());
  (void)hipGetDevice(&dev);
  bool found = false;
  for (JitInstance& j : plan->jit)
    if (j.expr.empty() && j.mt == c.sc.mt && j.nt == c.sc.nt && j.kw == c.sc.kw && j.moe == moe && j.device == dev) {
      j.fn = r.fn;
      found = true;
    }
  if (!found) plan->jit.push_back(JitInstance{c.sc.mt, c.sc.nt, c.sc.kw, dev, moe, r.fn, std::string()});
  if (info) {
    info->compile_ms = r.compile_ms;
    info->load_ms = r.load_ms;
    info->from_cache = r.from_cache;
    info->code_bytes = r.code_bytes;
    std::snprintf(info->key, sizeof info->key, "%s", r.key);
  }
  return ok();
}

qdg_status qdg_moe_align_capacity(int64_t T, int32_t top_k, int32_t E, int32_t block_m, int64_t* capacity) {
  if (!capacity) return fail(QDG_ERR_INVALID_ARG, "capacity is NULL");
  if (T < 0 || top_k < 1 || top_k > 32 || E < 1) return fail(QDG_ERR_INVALID_ARG, "bad T, top_k or E");
  if (E > 1024) return fail(QDG_ERR_UNSUPPORTED, "at most 1024 experts");
  if (block_m != 16 && block_m != 32 && block_m != 64 && block_m != 128)
    return fail(QDG_ERR_UNSUPPORTED, "block_m must be 16, 32, 64 or 128");
  if (T * top_k > (1 << 20)) return fail(QDG_ERR_UNSUPPORTED, "T*top_k above 2^20");
  *capacity = align_up(T * top_k + (int64_t)E * (block_m - 1), block_m);
  return ok();
}

qdg_status qdg_moe_align(const int32_t* topk_ids, int64_t T, int32_t top_k, int32_t E, int32_t block_m,
                         int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded, uint32_t* status,
                         void* stream) {
  int64_t cap = 0;
  qdg_status st = qdg_moe_align_capacity(T, top_k, E, block_m, &cap);
  if (st != QDG_OK) return st;
  if (!sorted_ids || !block_expert || !num_padded) return fail(QDG_ERR_INVALID_ARG, "NULL output");
  if (T > 0 && !topk_ids) return fail(QDG_ERR_INVALID_ARG, "topk_ids is NULL");
  if (!aligned(status, 4)) return fail(QDG_ERR_MISALIGNED, "status must be 4-byte aligned");
  return hip_status(launch_moe_align(topk_ids, T, top_k, E, block_m, cap, sorted_ids, block_expert, num_padded,
                                     status, (hipStream_t)stream),
                    "moe_align launch");
}

qdg_status qdg_moe_gemm(const qdg_plan* plan, const void* A, const float* a_scales, const void* packed,
                        const int32_t* sorted_ids, const int32_t* block_expert, const int32_t* num_padded,
                        int64_t T, int32_t block_m, int32_t a_per_pair, void* Y, void* workspace,
                        size_t ws_bytes, void* stream) {
  if (!plan) return fail(QDG_ERR_INVALID_ARG, "plan is NULL");
  if (plan->compute.kind != QDG_KIND_MOE) return fail(QDG_ERR_INVALID_ARG, "not a MoE plan");
  if (T < 0) return fail(QDG_ERR_INVALID_ARG, "T < 0");
  if (T == 0) return ok();
  if (block_m != 16 && block_m != 32 && block_m != 64 && block_m != 128)
    return fail(QDG_ERR_UNSUPPORTED, "grouped GEMM block_m must be 16, 32, 64 or 128");
  if (T * plan->compute.top_k > (1 << 20)) return fail(QDG_ERR_UNSUPPORTED, "T*top_k above 2^20");
  if (!A || !packed || !Y || !sorted_ids || !block_expert || !num_padded)
    return fail(QDG_ERR_INVALID_ARG, "NULL pointer");
  if (plan->fmt != FMT_W4A16 && plan->fmt != FMT_W8A16 && plan->fmt != FMT_NVFP4 && plan->fmt != FMT_W2A16 &&
      (plan->fmt == FMT_MXFP4 || plan->fmt == FMT_W4A4 || plan->fmt == FMT_MXFP4_I8 ||
       plan->layer.otype != QDG_O_I32) && !a_scales)
    return fail(QDG_ERR_INVALID_ARG, "activation scales are NULL");
  if (!aligned(A, 16)) return fail(QDG_ERR_MISALIGNED, "A must be 16-byte aligned");
  if (!aligned(packed, 256)) return fail(QDG_ERR_MISALIGNED, "packed must be 256-byte aligned");
  if (!aligned(Y, plan->layer.otype == QDG_O_BF16 ? 2 : 4))
    return fail(QDG_ERR_MISALIGNED, "Y must be aligned to its element size");
  return run(plan, A, a_scales, packed, Y, T, workspace, ws_bytes, (hipStream_t)stream, true, sorted_ids,
             block_expert, num_padded, T, block_m, a_per_pair ? 1 : 0);
}

static qdg_status moe_combine(const void* y, bool y_bf16, const float* w, int64_t T, int32_t top_k, int64_t n,
                              void* out, int32_t otype, void* stream) {
  if (T < 0 || n < 1 || top_k < 1 || top_k > 32) return fail(QDG_ERR_INVALID_ARG, "bad T, n or top_k");
  if (otype != QDG_O_BF16 && otype != QDG_O_F32) return fail(QDG_ERR_INVALID_ARG, "otype must be BF16 or F32");
  if (n % 4 != 0) return fail(QDG_ERR_UNSUPPORTED, "n must be a multiple of 4");
  if (T == 0) return ok();
  if (!y || !w || !out) return fail(QDG_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned(y, y_bf16 ? 8 : 16) || !aligned(out, 16))
    return fail(QDG_ERR_MISALIGNED, y_bf16 ? "y must be 8-byte and out 16-byte aligned" : "y and out must be 16-byte aligned");
  if (!aligned(w, 4)) return fail(QDG_ERR_MISALIGNED, "w must be 4-byte aligned");
  return hip_status(launch_moe_combine(y, y_bf16, w, T, top_k, n, out, otype, (hipStream_t)stream),
                    "moe_combine launch");
}

qdg_status qdg_moe_combine(const float* y, const float* w, int64_t T, int32_t top_k, int64_t n, void* out,
                           int32_t otype, void* stream) {
  return moe_combine(y, false, w, T, top_k, n, out, otype, stream);
}

qdg_status qdg_moe_combine_bf16(const void* y, const float* w, int64_t T, int32_t top_k, int64_t n, void* out,
                                int32_t otype, void* stream) {
  return moe_combine(y, true, w, T, top_k, n, out, otype, stream);
}

}  // extern "C"
