// LDS-tiled (large-M) W4A16 GEMM family for gfx950.
//
// The pages' library switches to a different, throughput-oriented pipeline
// for large batches (kinachrichten, "Wie die Architektur funktioniert"). Here
// the large-M path is MFMA-bound, so it is organised around MFMA issue:
//   * a 512-thread workgroup owns a 256 x 128 or 128 x 256 output tile; its
//     8 wavefronts (two per SIMD) each own a 64 x 64 tile computed as 2 x 2
//     blocks of 32 x 32 (v_mfma_f32_32x32x16_bf16). Per issued instruction
//     that form does twice the work of the 16 x 16 one, which leaves room for
//     the dequantization and scale VALU work to run under the matrix core
//     (measured: about six independent VALU ops hide under each 32 x 32 MFMA,
//     two under each 16 x 16 one);
//   * the K loop advances one 128-wide group per iteration. Everything the
//     next groups need -- the A tile, the A row sums, the packed weight units
//     and the scale records -- is copied global -> LDS with direct 16-byte
//     LDS loads into a three-stage ring of separate LDS arrays, so no
//     registers are held for prefetch. Every wave issues the same branch-free
//     copy sequence, so the wait before a group leaves the next group's
//     copies in flight; A rows are padded to 272 bytes so fragment reads are
//     bank-conflict-free;
//   * dequantization in registers as in the streaming family (bf16 128+u,
//     one v_and_or_b32 per dword); each MFMA chain of a group starts from
//     -(128+z) * rowsum(A) instead of zero, with the row sums computed (and,
//     when symmetric, pre-scaled by -136) once per call by rowsum_kernel, so
//     the only per-group epilogue is acc += s * P;
//   * the output tile is transposed through LDS so every global store writes
//     whole 16-byte row segments; the tile order is XCD-aware.
#ifndef __HIPCC_RTC__
#include <cstdio>
#include <type_traits>
#endif

#include "qdg_device.h"
#include "qdg_internal.h"

namespace qdg {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

// Row sums of A per 128-wide K group, times `factor`:
// out[g * m_pad + r] = factor * sum_k A[row(r)][128g + k], row(r) = r (dense;
// rows >= M give 0) or the gathered MoE row. Sixteen lanes take one
// (row, group) pair, 16 bytes each, so a wave reads 1 KiB of contiguous A
// (four consecutive groups of one row); the 16 partial sums meet by lane
// shuffles.
__global__ void rowsum_kernel(const uint16_t* __restrict__ A, const int* __restrict__ sorted_ids,
                              const int* __restrict__ num_padded, int top_k, int a_per_pair, int num_pairs,
                              int M, int K, int m_pad, float factor, float* __restrict__ out) {
  const int groups = K / 128;
  const int64_t pair = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 4;
  const int sub = threadIdx.x & 15;
  if (pair >= (int64_t)m_pad * groups) return;  // whole 16-lane groups
  const int r = (int)(pair / groups), g = (int)(pair % groups);
  int src = r;
  bool v = r < M;
  if (sorted_ids) {
    v = r < *num_padded;
    const int id = v ? sorted_ids[r] : num_pairs;
    v = id < num_pairs;
    src = v ? (a_per_pair ? id : id / top_k) : 0;
  }
  float s = 0.f;
  if (v) {
    const u32x4_t x = *(const u32x4_t*)(A + (size_t)src * K + (size_t)g * 128 + sub * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s += __builtin_bit_cast(float, (uint32_t)(x[j] << 16));
      s += __builtin_bit_cast(float, (uint32_t)(x[j] & 0xFFFF0000u));
    }
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) s += __shfl_xor(s, o, 16);
  if (sub == 0) out[(size_t)g * m_pad + r] = s * factor;
}

// Sum of the split-K partials in split order (deterministic), converted to
// the output type. partial is [nsplit][m_pad][n_pad] fp32.
__global__ void reduce_splits_kernel(const float* __restrict__ partial, void* __restrict__ Y, int M, int N,
                                     int m_pad, int n_pad, int nsplit, int otype) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // one 4-column chunk
  const int cpr = n_pad / 4;
  if (q >= (int64_t)M * cpr) return;
  const int row = (int)(q / cpr), c4 = (int)(q % cpr) * 4;
  if (c4 >= N) return;
  // four splits per step with their loads in flight together; the sum is
  // still taken in split order (deterministic)
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
  for (int sp0 = 0; sp0 < nsplit; sp0 += 4) {
    f32x4_t v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sp = sp0 + j < nsplit ? sp0 + j : nsplit - 1;
      v[j] = *(const f32x4_t*)(partial + ((size_t)sp * m_pad + row) * n_pad + c4);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (sp0 + j < nsplit) s = f32x4_t{s[0] + v[j][0], s[1] + v[j][1], s[2] + v[j][2], s[3] + v[j][3]};
  }
  for (int e = 0; e < 4 && c4 + e < N; ++e) {
    const size_t o = (size_t)row * N + c4 + e;
    if (otype == QDG_O_F32)
      ((float*)Y)[o] = s[e];
    else
      ((uint16_t*)Y)[o] = (uint16_t)f32_to_bf16_rne(s[e]);
  }
}

// Layout of one LDS stage (everything one K group needs):
//   A      BM rows of 272 bytes (128 bf16 + 16 bytes of padding: rows start
//          16 bytes apart modulo 128, so the 8 lanes served together by a
//          16-byte LDS read always hit distinct banks, and every fragment
//          address is one per-lane base plus an immediate offset)
//   RS     BM floats (row sums, pre-scaled), starting at the next 1 KiB
//          boundary after A (the A copies move whole 1 KiB spans), in a slot
//          one whole-wave copy fills: 256 bytes (4 per lane) for up to 64
//          rows, else at least 1 KiB (16 per lane); the small slot is what
//          lets three stages of 64 x 512 tiles fit in the 160 KiB
//   W      BN/16 packed weight units of UB bytes (1 KiB for 4-bit codes, 2 KiB
//          for int8; tile-major)
//   S      BN/16 x 16 scale records of 8 bytes
template <int BM, int BN, int UB = 1024>
struct Stage {
  static constexpr int ROW = 272;
  static constexpr int A = 0;
  static constexpr int A_SLOTS = BM * ROW / 16;  // 16-byte slots, 17 per row
  // whole 1 KiB copies fill A (the last one may run past BM rows)
  static constexpr int RS = (BM * ROW + 1023) / 1024 * 1024;
  static constexpr bool RS_SMALL = BM <= 64;  // 4-byte copies into a 256-byte slot
  static constexpr int W = RS + (RS_SMALL ? 256 : BM * 4 > 1024 ? BM * 4 : 1024);
  static constexpr int S = W + (BN / 16) * UB;
  static constexpr int BYTES = S + (BN / 16) * 128;
};

// Issue the global -> LDS copies of group g into `st` (direct 16-byte LDS
// loads: lane l of a wave instruction writes bytes 16l..16l+15 of a 1 KiB
// LDS span). Global addresses are a wave-uniform base plus a 32-bit lane
// offset fixed for the whole K loop. Kept out of lambdas: a device-only
// builtin inside an (implicitly host+device) lambda makes the host pass drop
// the kernel.
// Packed N tile behind stage tile t of a workgroup whose tiles start at
// `base`. With the SiLU*mul epilogue (BN / 16 stage tiles) the first half are
// gate tiles base.. and the second half the matching up tiles G + base..
// (G = I / 16); tiles past the layer re-read the last one and are never
// stored.
template <int BN>
__device__ __forceinline__ int stage_tile(const GemmArgs& p, int base, int t) {
  constexpr int HALF = BN / 32;
  if (p.epi == QDG_EPI_SILU_MUL) {
    const int G = p.ntiles / 2;
    const int j = min(base + t % HALF, G - 1);
    return t < HALF ? j : G + j;
  }
  return min(base + t, p.ntiles - 1);
}

template <int BM, int BN, int NW, bool RS = true, int UB = 1024>
__device__ __forceinline__ void load_stage(char* st, const char* a_g, const uint32_t* a_off, const GemmArgs& p,
                                           const uint8_t* wbase, const uint8_t* sbase, uint32_t s_off,
                                           int wg_tile0, int wave, int lane, int mb, int g) {
  // Every wave issues the same copies without branches, so that a wait on
  // the copy count is exact for every wave and the compiler can tell which
  // stage each copy writes. Surplus copies repeat another wave's copy (the
  // same bytes to the same place).
  using L = Stage<BM, BN, UB>;
  constexpr int A_INST = (L::A_SLOTS + 63) / 64;
  constexpr int WC = UB >= 1024 ? UB / 1024 : 1;  // 1 KiB copies per unit
  static_assert((BN / 16) * WC % NW == 0, "whole weight copies per wave");
  const char* ag = a_g + (size_t)g * 256;
#pragma unroll
  for (int r = 0; r < (A_INST + NW - 1) / NW; ++r) {
    const int i = min(r * NW + wave, A_INST - 1);
    __builtin_amdgcn_global_load_lds(ag + a_off[r], (lds_void*)(st + L::A + i * 1024), 16, 0, 0);
  }
  if constexpr (UB == 512) {
    // 2-bit units: two copies of 256 bytes (4 per lane) per unit
    static_assert((BN / 16) * 2 % NW == 0, "whole weight copies per wave");
#pragma unroll
    for (int r = 0; r < (BN / 16) * 2 / NW; ++r) {
      const int ci = r * NW + wave;
      const int t = ci / 2, part = ci % 2;
      const int tile = stage_tile<BN>(p, wg_tile0, t);
      __builtin_amdgcn_global_load_lds(wbase + ((size_t)tile * p.groups + g) * UB + part * 256 + lane * 4,
                                       (lds_void*)(st + L::W + t * UB + part * 256), 4, 0, 0);
    }
  } else {
#pragma unroll
    for (int r = 0; r < (BN / 16) * WC / NW; ++r) {
      const int ci = r * NW + wave;
      const int t = ci / WC, part = ci % WC;
      const int tile = stage_tile<BN>(p, wg_tile0, t);
      __builtin_amdgcn_global_load_lds(wbase + ((size_t)tile * p.groups + g) * UB + part * 1024 + lane * 16,
                                       (lds_void*)(st + L::W + t * UB + part * 1024), 16, 0, 0);
    }
  }
  // scale records: BN / 128 copies of 1 KiB, copy wave % (BN / 128) per wave
  // (int8 weights have one scale per channel, applied in the epilogue)
  if constexpr (UB != 2048)
    __builtin_amdgcn_global_load_lds(sbase + (size_t)g * 128 + s_off,
                                     (lds_void*)(st + L::S + (wave % (BN / 128)) * 1024), 16, 0, 0);
  // row sums: one whole-wave copy per wave; lanes past the block's rows
  // repeat rows into the unused rest of the slot
  if constexpr (RS) {
    if constexpr (L::RS_SMALL) {
      const float* rs = p.rowsum + (size_t)g * p.m_pad + mb * BM + lane % BM;
      __builtin_amdgcn_global_load_lds(rs, (lds_void*)(st + L::RS), 4, 0, 0);
    } else {
      static_assert(BM / 4 <= 64, "one copy of row sums");
      const char* rs = (const char*)(p.rowsum + (size_t)g * p.m_pad + mb * BM) + (lane % (BM / 4)) * 16;
      __builtin_amdgcn_global_load_lds(rs, (lds_void*)(st + L::RS), 16, 0, 0);
    }
  }
}

// One K group for a 64 x 64 wave tile: unpack the wave's 4 weight tiles once,
// then for each 16-row A tile run the four N-tile MFMA chains interleaved
// (each chain seeded with -(128+z) * rowsum) and fold them into the
// accumulators with the group scales. N tiles past the end of the layer hold
// duplicate data: computed like the others and never stored.
// MTR: the row tiles run (grouped MoE: fewer when the wave's later rows are
// all padding).
template <bool ASYM, int BM, int BN, int MTW, int MTR = MTW>
__device__ __forceinline__ void tile_group(const char* st, int a_lane, int w_lane, int s_lane, int rs_lane,
                                           uint32_t um, uint32_t ue, f32x4_t (&acc)[MTW][4]) {
  using L = Stage<BM, BN>;
  u32x4_t bp[4];
  u32x4_t bw[4][4];
  float sc[4], negz[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    bp[t] = *(const u32x4_t*)(st + w_lane + t * 1024);
    const u32x2_t rec = *(const u32x2_t*)(st + s_lane + t * 128);
    sc[t] = bits_as<float>(rec.x);
    negz[t] = __builtin_bit_cast(float, (rec.y & 0xFFFFu) << 16);  // -(128+z)
  }
#pragma unroll
  for (int mt = 0; mt < MTR; ++mt) {
    u32x4_t a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = *(const u32x4_t*)(st + a_lane + mt * 16 * L::ROW + j * 16);
    const f32x4_t rs = *(const f32x4_t*)(st + rs_lane + mt * 64);
    f32x4_t pacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if constexpr (ASYM)
        pacc[t] = f32x4_t{negz[t] * rs[0], negz[t] * rs[1], negz[t] * rs[2], negz[t] * rs[3]};
      else
        pacc[t] = rs;  // row sums pre-scaled by -136
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // unpack step j of every tile right before its first use, so the
      // first MFMAs of the group start early
      if (mt == 0) {
#pragma unroll
        for (int t = 0; t < 4; ++t) bw[t][j] = unpack_u4_bf16_offset128(bp[t][j], um, ue);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) pacc[t] = mfma_bf16(a[j], bw[t][j], pacc[t]);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[mt][t][i] = __builtin_fmaf(sc[t], pacc[t][i], acc[mt][t][i]);
  }
}

// One K group for a 64 x 64 wave tile as 2 x 2 blocks of 32 x 32 outputs
// (v_mfma_f32_32x32x16_bf16). Each MFMA does twice the work of the 16 x 16
// form for the same issue cost, so the unpack and scale VALU work of the
// group fits under the matrix core. Any assignment of the group's 128 K
// values to the eight K steps works as long as A and W agree: lane half h
// takes, at step s, dword s % 4 of unit quarter h + 2 * (s / 4), i.e. K
// values 32 (h + 2 (s / 4)) + 8 (s % 4) .. +7, and reads the same eight
// A values.
// RB = 1 runs only the first row block (grouped MoE: the wave's rows 32..63
// are all padding).
template <bool ASYM, int BM, int BN, int RB = 2>
__device__ __forceinline__ void tile_group32(const char* st, int a_lane, int w_lane, int s_lane, int rs_lane,
                                             uint32_t um, uint32_t ue, f32x16_t (&acc)[2][2]) {
  using L = Stage<BM, BN>;
  u32x4_t bp[2][2];  // [column block][quarter h, quarter h + 2]
  float sc[2], negz[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
    for (int q = 0; q < 2; ++q) bp[cb][q] = *(const u32x4_t*)(st + w_lane + cb * 2048 + q * 512);
    const u32x2_t rec = *(const u32x2_t*)(st + s_lane + cb * 256);
    sc[cb] = bits_as<float>(rec.x);
    negz[cb] = __builtin_bit_cast(float, (rec.y & 0xFFFFu) << 16);  // -(128+z)
  }
  // each chain starts from the row sums of its rows (times -(128+z))
  f32x16_t pacc[2][2];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    f32x4_t r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = *(const f32x4_t*)(st + rs_lane + rb * 128 + q * 32);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) pacc[rb][cb][i] = ASYM ? negz[cb] * r[i / 4][i % 4] : r[i / 4][i % 4];
  }
  // the A fragments of four steps are read together before their MFMAs (the
  // reads complete in order, so each MFMA waits only for its own): left to
  // itself the scheduler reads each step's fragment of the second row block
  // into the same registers right before its MFMAs, exposing one LDS
  // latency per step (all eight steps at once would need more registers
  // than two waves per SIMD have)
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) {
    u32x4_t a[4][2];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        a[s][rb] = *(const u32x4_t*)(st + a_lane + rb * 32 * L::ROW + hs * 128 + s * 16);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4_t b[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) b[cb] = unpack_u4_bf16_offset128(bp[cb][hs][s], um, ue);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) pacc[rb][cb] = mfma_bf16_32(a[s][rb], b[cb], pacc[rb][cb]);
    }
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rb][cb][i] = __builtin_fmaf(sc[cb], pacc[rb][cb][i], acc[rb][cb][i]);
}

// W2A16 (2-bit codes, fp16 group scales, zero points 0..3) in the same 2 x 2
// blocks: the 4-bit path with 512-byte units. A lane of quarter q = s / 4 at
// step s reads unit lane h + 2q, whose dword (s % 4) / 2 holds that step's
// eight codes in the fields 4 (s % 2) .. 4 (s % 2) + 3 (low and high half);
// each bf16 pair 128 + u is one shift and one v_and_or_b32 (um = 0x00030003),
// and each chain starts from -(128 + z) * rowsum(A).
template <int BM, int BN>
__device__ __forceinline__ void tile_group32_w2(const char* st, int a_lane, int w2_lane, int s_lane, int rs_lane,
                                                uint32_t um, uint32_t ue, f32x16_t (&acc)[2][2]) {
  using L = Stage<BM, BN, 512>;
  u32x2_t bp[2][2];  // [column block][quarter h, quarter h + 2]
  float sc[2], negz[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
    for (int q = 0; q < 2; ++q) bp[cb][q] = *(const u32x2_t*)(st + w2_lane + cb * 1024 + q * 256);
    const u32x2_t rec = *(const u32x2_t*)(st + s_lane + cb * 256);
    sc[cb] = bits_as<float>(rec.x);
    negz[cb] = __builtin_bit_cast(float, (rec.y & 0xFFFFu) << 16);  // -(128+z)
  }
  f32x16_t pacc[2][2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    f32x4_t r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = *(const f32x4_t*)(st + rs_lane + rb * 128 + q * 32);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) pacc[rb][cb][i] = negz[cb] * r[i / 4][i % 4];
  }
  // A fragments of four steps read together before their MFMAs (as in
  // tile_group32)
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) {
    u32x4_t a[4][2];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        a[s][rb] = *(const u32x4_t*)(st + a_lane + rb * 32 * L::ROW + hs * 128 + s * 16);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4_t b[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const uint32_t x = bp[cb][hs][s / 2];
#pragma unroll
        for (int m = 0; m < 4; ++m) b[cb][m] = ((x >> (8 * (s % 2) + 2 * m)) & um) | ue;
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) pacc[rb][cb] = mfma_bf16_32(a[s][rb], b[cb], pacc[rb][cb]);
    }
  }
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rb][cb][i] = __builtin_fmaf(sc[cb], pacc[rb][cb][i], acc[rb][cb][i]);
}

// NVFP4 weights (E2M1 with E4M3 scales per 16 K) in the same 2 x 2 blocks
// of 32 x 32: each weight is converted, multiplied by its block scale (both
// exact) and packed to bf16, so the MFMAs accumulate straight into the
// result with no per-group epilogue and no row sums. The scale records hold,
// per unit lane (c, col) of the streaming layout, the E4M3 codes of that
// lane's two 16-blocks; a lane of quarter q = s / 4 at step s reads unit
// lane h + 2q, whose dword s % 4 lies in its block (s % 4) / 2.
template <int BM, int BN>
__device__ __forceinline__ void tile_group32_nv(const char* st, int a_lane, int w_lane, int sv_lane,
                                                f32x16_t (&acc)[2][2]) {
  using L = Stage<BM, BN>;
  u32x4_t bp[2][2];
  uint32_t rec[2][2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      bp[cb][q] = *(const u32x4_t*)(st + w_lane + cb * 2048 + q * 512);
      rec[cb][q] = *(const uint16_t*)(st + sv_lane + cb * 256 + q * 64);
    }
  // A fragments of four steps read together before their MFMAs (as in
  // tile_group32)
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) {
    u32x4_t a[4][2];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        a[s][rb] = *(const u32x4_t*)(st + a_lane + rb * 32 * L::ROW + hs * 128 + s * 16);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4_t b[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        b[cb] = e2m1x8_scaled_bf16(bp[cb][hs][s], e4m3_to_f32((rec[cb][hs] >> (8 * (s / 2))) & 0xFFu));
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = mfma_bf16_32(a[s][rb], b[cb], acc[rb][cb]);
    }
  }
}

// W8A16 (int8 weights, one fp32 scale per channel) in the same blocks: each
// int8 q enters the MFMA as the bf16 integer q + 128 and each group's chains
// start from the row sums of A pre-scaled by -128, so a group adds exactly
// sum A * q; the channel scale is applied in the epilogue. Unit lane (c, col)
// holds K 32c..32c+15 in its first 16-byte chunk and 32c+16..32c+31 in its
// second (1 KiB further on); step s reads unit lane h + 2 (s / 4), chunk
// (s % 4) / 2, dwords 2 (s % 2) and 2 (s % 2) + 1.
template <int BM, int BN>
__device__ __forceinline__ void tile_group32_w8(const char* st, int a_lane, int w8_lane, int rs_lane,
                                                f32x16_t (&acc)[2][2]) {
  using L = Stage<BM, BN, 2048>;
  f32x16_t pacc[2][2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    f32x4_t r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = *(const f32x4_t*)(st + rs_lane + rb * 128 + q * 32);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) pacc[rb][cb][i] = r[i / 4][i % 4];
  }
  // A fragments and weight chunks of four steps read together before their
  // MFMAs (as in tile_group32)
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) {
    u32x4_t a[4][2], ch[2][2];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        a[s][rb] = *(const u32x4_t*)(st + a_lane + rb * 32 * L::ROW + hs * 128 + s * 16);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        ch[cb][j] = *(const u32x4_t*)(st + w8_lane + cb * 2 * 2048 + hs * 512 + j * 1024);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4_t b[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const u32x4_t c4 = ch[cb][s / 2];
        b[cb] = i8x8_bf16_offset128(s % 2 ? c4.z : c4.x, s % 2 ? c4.w : c4.y);
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) pacc[rb][cb] = mfma_bf16_32(a[s][rb], b[cb], pacc[rb][cb]);
    }
  }
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rb][cb][i] += pacc[rb][cb][i];
}

template <int V>
struct IntC {
  static constexpr int value = V;
};

template <bool ASYM, int WAVES_M, int WAVES_N, int WTM, int NS, bool MOE, bool NV = false, bool W8 = false,
          bool W2 = false>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void tile_gemm_kernel(const GemmArgs p, int m_blocks,
                                                                           int n_blocks) {
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int BM = WTM * WAVES_M, BN = 64 * WAVES_N;
  constexpr int MTW = WTM / 16;  // 16-row tiles per wave
  constexpr bool M32 = WTM == 64;  // 64 x 64 wave tiles run 32 x 32 MFMA blocks
  constexpr int UB = W8 ? 2048 : W2 ? 512 : 1024;  // bytes per weight unit
  using L = Stage<BM, BN, UB>;
  constexpr int A_INST = (L::A_SLOTS + 63) / 64;
  constexpr int A_PER_WAVE = (A_INST + NW - 1) / NW;
  // copies every wave issues per stage (A, weight units, scale records, row
  // sums); waiting for the count to drop to this leaves the next stage in
  // flight
  constexpr int VM_NEXT =
      A_PER_WAVE + (BN / 16) * (W2 ? 2 : UB / 1024) / NW + (W8 ? 0 : 1) + (NV ? 0 : 1);
  static_assert(!NV || M32, "NVFP4 runs the 64 x 64 wave tiles");
  static_assert(!W8 || (M32 && !NV), "W8A16 runs the 64 x 64 wave tiles");
  static_assert(!W2 || (M32 && ASYM && !NV && !W8), "W2A16 runs the 64 x 64 wave tiles with zero points");
  static_assert(NS == 2 || NS == 3, "two or three stages");
  // The stages are separate LDS objects (not one dynamic array) so that the
  // compiler can tell a copy into one stage from a read of another: reads of
  // a stage then wait only for that stage's copies.
  __shared__ __attribute__((aligned(16))) char st0[L::BYTES];
  __shared__ __attribute__((aligned(16))) char st1[L::BYTES];
  __shared__ __attribute__((aligned(16))) char st2[NS == 3 ? L::BYTES : 16];
  char* const stage[3] = {st0, st1, st2};

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int c = lane >> 4, col = lane & 15;

  // XCD-aware tile order: consecutive workgroup ids land on different XCDs,
  // so XCD x takes the x-th eighth of the tile order; that order walks 4 x 8
  // blocks of tiles, so the tiles an XCD runs at once share row blocks of A
  // and column blocks of W in its L2 (grouped MoE: moe_tile_order)
  int mb, nb;
  if constexpr (MOE) {
    moe_tile_order(n_blocks, mb, nb);
  } else {
    const int total = m_blocks * n_blocks;
    int lin = blockIdx.x;
    if (total % 8 == 0) lin = (lin % 8) * (total / 8) + lin / 8;
    if (m_blocks % 4 == 0 && n_blocks % 8 == 0) {
      const int sb = lin / 32, w = lin % 32;
      mb = (sb / (n_blocks / 8)) * 4 + w / 8;
      nb = (sb % (n_blocks / 8)) * 8 + w % 8;
    } else {
      mb = lin / n_blocks;
      nb = lin % n_blocks;
    }
  }
  // split-K: this workgroup reduces K groups [g0, g1) of the tile
  const int split = blockIdx.y, nsplit = gridDim.y;
  const int g0 = (int)(((int64_t)split * p.groups) / nsplit);
  const int g1 = (int)(((int64_t)(split + 1) * p.groups) / nsplit);

  int expert = 0;
  if constexpr (MOE) {
    if (mb * BM >= *p.num_padded) return;
    expert = p.block_expert[mb];
  }
  const uint8_t* wbase = p.packed + (size_t)expert * p.expert_stride;
  // NVFP4: the expert's tensor scale leads its scale region, the records follow
  const uint8_t* sbase = wbase + p.s_offset + (NV ? 256 : 0);
  const int groups = p.groups;
  // SiLU*mul (MoE gate+up): 16 stage tiles = 8 gate + 8 up tiles, i.e. 8
  // output tiles per workgroup
  const bool silu = MOE && !NV && !W8 && p.epi == QDG_EPI_SILU_MUL;  // W4A16 only
  static_assert(!MOE || WAVES_N % 2 == 0, "the SiLU*mul pairing splits the waves' columns in halves");
  const int wg_tile0 = silu ? nb * (BN / 32) : nb * (BN / 16);

  // A copy plan: slot q = 64 i + lane of the padded tile is row q / 17,
  // 16-byte chunk q % 17 (chunk 16 is padding: it re-reads chunk 0)
  uint32_t a_off[A_PER_WAVE];
#pragma unroll
  for (int r = 0; r < A_PER_WAVE; ++r) {
    const int q = min(r * NW + wave, A_INST - 1) * 64 + lane;
    const int row = min(q / 17, BM - 1), ch = q % 17;
    const int grow = mb * BM + row;
    int src;
    if constexpr (MOE) {
      const int id = p.sorted_ids[grow];
      src = id < p.num_pairs ? (p.a_per_pair ? id : id / p.top_k) : 0;
    } else {
      src = grow < p.M ? grow : p.M - 1;
    }
    a_off[r] = (uint32_t)src * (uint32_t)(p.K * 2) + (uint32_t)(ch < 16 ? ch : 0) * 16;
  }
  // scale records: lane l fetches 16 bytes (l % 8) of tile 8r + l / 8
  // scale records: lane l fetches 16 bytes (l % 8) of tile 8 r + l / 8 of
  // copy r = wave % (BN / 128)
  uint32_t s_off;
  {
    const int s_tile = stage_tile<BN>(p, wg_tile0, 8 * (wave % (BN / 128)) + (lane >> 3));
    s_off = (uint32_t)s_tile * (uint32_t)groups * 128u + (lane & 7) * 16;
  }

  // per-lane LDS bases of the fragment reads (byte offsets inside a stage);
  // 64 x 64 wave tiles use 32 x 32 blocks: lane half h = lane / 32 reads
  // row / column lane % 32 (column block b covers units 4 wn + 2 b + 0..1)
  const int h = lane >> 5, l32 = lane & 31;
  const int a_lane = M32 ? L::A + (wm * WTM + l32) * L::ROW + h * 64 : L::A + (wm * WTM + col) * L::ROW + c * 64;
  const int w_lane = M32 ? L::W + (wn * 4 + (l32 >> 4)) * 1024 + (h * 16 + col) * 16 : L::W + (wn * 4) * 1024 + lane * 16;
  const int s_lane = M32 ? L::S + (wn * 4 + (l32 >> 4)) * 128 + col * 8 : L::S + (wn * 4) * 128 + col * 8;
  const int rs_lane = M32 ? L::RS + (wm * WTM + 4 * h) * 4 : L::RS + (wm * WTM + 4 * c) * 4;
  const int sv_lane = L::S + (wn * 4 + (l32 >> 4)) * 128 + (h * 16 + col) * 2;  // NVFP4 scale records
  const int w8_lane = L::W + (wn * 4 + (l32 >> 4)) * 2048 + (h * 16 + col) * 16;  // W8A16 units
  const int w2_lane = L::W + (wn * 4 + (l32 >> 4)) * 512 + (h * 16 + col) * 8;    // W2A16 units

  // one unpack constant in a VGPR, the other in an SGPR: lets each unpacked
  // dword be a single v_and_or_b32 (VOP3 reads at most one scalar operand)
  uint32_t um;
  asm volatile("v_mov_b32 %0, %1" : "=v"(um) : "s"(p.unpack_mask));
  const uint32_t ue = p.unpack_exp;

  f32x4_t acc[MTW][4];
  f32x16_t acc32[2][2];
  if constexpr (M32) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc32[rb][cb][i] = 0.f;
  } else {
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[mt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const char* a_g = (const char*)p.A;
  // NS-stage ring. Full rounds of NS groups run unrolled with constant stage
  // indices; each group issues the copies of the group NS - 1 ahead (clamped
  // to the last group: past the range they re-read it into a stage nobody
  // reads again), so with three stages the wait before a group leaves the
  // next group's copies in flight. The last partial round waits for all
  // copies.
  if (g0 < g1) {
#pragma unroll
    for (int q = 0; q < NS - 1; ++q)
      load_stage<BM, BN, NW, !NV, UB>(stage[q], a_g, a_off, p, wbase, sbase, s_off, wg_tile0, wave, lane, mb,
                             min(g0 + q, g1 - 1));
  }
  // The K loop, instantiated per count of the wave's row blocks that hold
  // real rows (RB = 1: only the first half): a grouped MoE wave whose second
  // half of rows (32..63 of a 64-row wave tile, 16..31 of a 32-row one) is
  // all padding (an expert's real entries lead its blocks, so the entry at
  // the half's first row tells) skips their fragment reads and MFMAs. Both
  // instances run the same barriers, so the waves of one workgroup may take
  // different ones.
  auto k_loop = [&](auto rb_count) __attribute__((always_inline)) {
    constexpr int RB = decltype(rb_count)::value;
    int gb = g0;
    for (; gb + NS <= g1; gb += NS) {
#pragma unroll
      for (int cur = 0; cur < NS; ++cur) {
        // this wave's copies of group gb+cur are done once at most the copies
        // of one later group remain in flight (copies complete in order)
        if constexpr (NS == 3)
          __builtin_amdgcn_s_waitcnt((VM_NEXT & 15) | (7 << 4) | (15 << 8) | ((VM_NEXT >> 4) << 14));
        else
          __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        // every wave's copies of the group landed and every wave is done with
        // the previous group's stage. A bare s_barrier: __syncthreads would also
        // wait for the copies in flight.
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        asm volatile("s_barrier" ::: "memory");
        load_stage<BM, BN, NW, !NV, UB>(stage[(cur + NS - 1) % NS], a_g, a_off, p, wbase, sbase, s_off, wg_tile0, wave, lane,
                               mb, min(gb + cur + NS - 1, g1 - 1));
        if constexpr (NV)
          tile_group32_nv<BM, BN>(stage[cur], a_lane, w_lane, sv_lane, acc32);
        else if constexpr (W8)
          tile_group32_w8<BM, BN>(stage[cur], a_lane, w8_lane, rs_lane, acc32);
        else if constexpr (W2)
          tile_group32_w2<BM, BN>(stage[cur], a_lane, w2_lane, s_lane, rs_lane, um, ue, acc32);
        else if constexpr (M32)
          tile_group32<ASYM, BM, BN, RB>(stage[cur], a_lane, w_lane, s_lane, rs_lane, um, ue, acc32);
        else
          tile_group<ASYM, BM, BN, MTW, RB == 2 ? MTW : 1>(stage[cur], a_lane, w_lane, s_lane, rs_lane, um, ue, acc);
      }
    }
#pragma unroll
    for (int cur = 0; cur < NS - 1; ++cur) {
      if (gb + cur < g1) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if constexpr (NV)
          tile_group32_nv<BM, BN>(stage[cur], a_lane, w_lane, sv_lane, acc32);
        else if constexpr (W8)
          tile_group32_w8<BM, BN>(stage[cur], a_lane, w8_lane, rs_lane, acc32);
        else if constexpr (W2)
          tile_group32_w2<BM, BN>(stage[cur], a_lane, w2_lane, s_lane, rs_lane, um, ue, acc32);
        else if constexpr (M32)
          tile_group32<ASYM, BM, BN, RB>(stage[cur], a_lane, w_lane, s_lane, rs_lane, um, ue, acc32);
        else
          tile_group<ASYM, BM, BN, MTW, RB == 2 ? MTW : 1>(stage[cur], a_lane, w_lane, s_lane, rs_lane, um, ue, acc);
      }
    }
  };
  if constexpr (MOE && M32 && !NV && !W8 && !W2) {
    if (p.sorted_ids[mb * BM + wm * WTM + 32] >= p.num_pairs)
      k_loop(IntC<1>{});
    else
      k_loop(IntC<2>{});
  } else if constexpr (MOE && !M32 && MTW == 2) {
    // 32-row wave tiles of 16 x 16 MFMAs: rows 16..31 all padding
    if (p.sorted_ids[mb * BM + wm * WTM + 16] >= p.num_pairs)
      k_loop(IntC<1>{});
    else
      k_loop(IntC<2>{});
  } else {
    k_loop(IntC<2>{});
  }

  // ---- epilogue: per wave, transpose each 16 x 64 strip through LDS so that
  // every lane stores whole 16-byte row segments
  __builtin_amdgcn_s_waitcnt(0);  // the trailing copies have landed
  __syncthreads();                 // everyone is done with the stages
  if (silu) {
    // gate columns sit in waves wn < WAVES_N / 2 and the matching up columns
    // in waves wn + WAVES_N / 2: per 16-row strip every wave parks its fp32
    // values in LDS, then the gate waves form silu(G) * U and store I-wide rows
    float* own = (float*)(st0 + wave * (16 * 64 * 4));
    const float* up = (const float*)(st0 + (wave + WAVES_N / 2) * (16 * 64 * 4));
    const int I = p.N / 2;
    const bool f32o = p.otype == QDG_O_F32;
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) {
      if constexpr (M32) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              own[(8 * q + 4 * h + i) * 64 + cb * 32 + l32] = acc32[mt / 2][cb][(2 * (mt % 2) + q) * 4 + i];
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) own[(4 * c + i) * 64 + t * 16 + col] = acc[mt][t][i];
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (wn < WAVES_N / 2) {
        for (int chunk = lane; chunk < 16 * 16; chunk += 64) {  // 16 rows x 16 chunks of 4 columns
          const int r = chunk >> 4, cc = chunk & 15;
          const int lrow = mb * BM + wm * WTM + mt * 16 + r;
          const int id = p.sorted_ids[lrow];
          const int n0 = wg_tile0 * 16 + wn * 64 + cc * 4;
          if (id >= p.num_pairs || n0 >= I) continue;
          const f32x4_t g4 = *(const f32x4_t*)(own + r * 64 + cc * 4);
          const f32x4_t u4 = *(const f32x4_t*)(up + r * 64 + cc * 4);
          float hv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) hv[e] = g4[e] / (1.f + expf(-g4[e])) * u4[e];
          if (f32o) {
            *(f32x4_t*)((float*)p.Y + (size_t)id * I + n0) = f32x4_t{hv[0], hv[1], hv[2], hv[3]};
          } else {
            u32x2_t pk;
            pk.x = f32_to_bf16_rne(hv[0]) | (f32_to_bf16_rne(hv[1]) << 16);
            pk.y = f32_to_bf16_rne(hv[2]) | (f32_to_bf16_rne(hv[3]) << 16);
            *(u32x2_t*)((uint16_t*)p.Y + (size_t)id * I + n0) = pk;
          }
        }
      }
      __syncthreads();  // the strips are rewritten for the next 16 rows
    }
    return;
  }
  // split-K: each split stores its fp32 partial tile row-major into the
  // workspace ([split][m_pad][n_pad]); reduce_splits_kernel sums them
  const bool to_partial = nsplit > 1;
  const int n_pad = n_blocks * BN;
  const bool f32out = to_partial || p.otype == QDG_O_F32;
  char* strip = st0 + wave * (16 * 64 * 4);
  static_assert(NW * 16 * 64 * 4 <= L::BYTES, "epilogue strips fit one stage");
  const int nbase = (wg_tile0 + wn * 4) * 16;
  const int esz = f32out ? 4 : 2;  // bytes per output element
  const float tscale = NV ? *(const float*)(wbase + p.s_offset) : 1.0f;  // NVFP4 tensor scale
  float csc[2] = {1.0f, 1.0f};  // W8A16: the channel scales of this lane's two columns
  if constexpr (W8) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int n = nbase + cb * 32 + l32;
      csc[cb] = n < p.N ? ((const float*)(wbase + p.s_offset))[n] : 0.f;
    }
  }
  const int cpr = 64 * esz / 16;   // 16-byte chunks per strip row
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt) {
    if constexpr (M32) {
      // rows 16 mt .. 16 mt + 15 of the wave tile: block mt / 2, result
      // elements i with i / 4 = 2 (mt % 2) + q
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = acc32[mt / 2][cb][(2 * (mt % 2) + q) * 4 + i];
            if constexpr (NV) v *= tscale;
            if constexpr (W8) v *= csc[cb];
            const int e = (8 * q + 4 * h + i) * 64 + cb * 32 + l32;
            if (f32out)
              ((float*)strip)[e] = v;
            else
              ((uint16_t*)strip)[e] = (uint16_t)f32_to_bf16_rne(v);
          }
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = (4 * c + i) * 64 + t * 16 + col;
          if (f32out)
            ((float*)strip)[e] = acc[mt][t][i];
          else
            ((uint16_t*)strip)[e] = (uint16_t)f32_to_bf16_rne(acc[mt][t][i]);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    for (int chunk = lane; chunk < 16 * cpr; chunk += 64) {
      const int r = chunk / cpr, cc = chunk % cpr;
      const int lrow = mb * BM + wm * WTM + mt * 16 + r;
      int yrow = lrow;
      bool v;
      if constexpr (MOE) {
        const int id = p.sorted_ids[lrow];
        v = id < p.num_pairs;
        yrow = id;
      } else {
        v = lrow < p.M;
      }
      const int per = 16 / esz;  // elements per chunk
      const int n0 = nbase + cc * per;
      const u32x4_t val = *(const u32x4_t*)(strip + r * 64 * esz + cc * 16);
      if (to_partial) {
        float* dst = (float*)p.partial + ((size_t)split * p.m_pad + lrow) * n_pad + n0;
        *(u32x4_t*)dst = val;
        continue;
      }
      if (v && n0 < p.N) {
        char* dst = (char*)p.Y + ((size_t)yrow * p.N + n0) * esz;
        if (n0 + per <= p.N && ((uintptr_t)dst & 15) == 0) {
          *(u32x4_t*)dst = val;
        } else if (f32out) {
          for (int e = 0; e < per && n0 + e < p.N; ++e) ((uint32_t*)dst)[e] = val[e];
        } else {
          for (int e = 0; e < per && n0 + e < p.N; ++e)
            ((uint16_t*)dst)[e] = (uint16_t)(val[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

#ifndef __HIPCC_RTC__  // host launchers
template <bool ASYM, int WAVES_M, int WAVES_N, int WTM, bool MOE, bool NV = false, bool W8 = false,
          bool W2 = false>
hipError_t launch_tile_cfg(const GemmArgs& a, int m_blocks, int nsplit, hipStream_t s, KernelLaunch* d) {
  constexpr int BM = WTM * WAVES_M, BN = 64 * WAVES_N;
  // as many stages as fit in the 160 KiB of LDS (3 for 128 x 256, 16 x 512,
  // 32 x 512 and 64 x 512, 2 for 256 x 128 and int8 units)
  constexpr int NS = 3 * Stage<BM, BN, W8 ? 2048 : W2 ? 512 : 1024>::BYTES <= 160 * 1024 ? 3 : 2;
  const int n_blocks = (a.ntiles + BN / 16 - 1) / (BN / 16);
  // grouped MoE: whole groups of 8 expert blocks (the order of moe_tile_order)
  const int grid_m = MOE ? moe_grid_blocks(m_blocks) : m_blocks;
  if (d) {
    auto b = [](bool v) { return v ? "true" : "false"; };
    d->src = JIT_SRC_TILE;
    std::snprintf(d->expr, sizeof d->expr, "qdg::tile_gemm_kernel<%s, %d, %d, %d, %d, %s, %s, %s, %s>", b(ASYM),
                  WAVES_M, WAVES_N, WTM, NS, b(MOE), b(NV), b(W8), b(W2));
    d->grid[0] = (unsigned)(grid_m * n_blocks);
    d->grid[1] = (unsigned)nsplit;
    d->grid[2] = 1;
    d->block = 64 * WAVES_M * WAVES_N;
    d->mn_args = true;
    d->m_blocks = m_blocks;
    d->n_blocks = n_blocks;
    return hipSuccess;
  }
  hipLaunchKernelGGL((tile_gemm_kernel<ASYM, WAVES_M, WAVES_N, WTM, NS, MOE, NV, W8, W2>), dim3(grid_m * n_blocks, nsplit),
                     dim3(64 * WAVES_M * WAVES_N), 0, s, a, m_blocks, n_blocks);
  return hipGetLastError();
}

#endif  // __HIPCC_RTC__
}  // namespace

#ifndef __HIPCC_RTC__  // host launchers
// Instances: (block_m, block_n, waves) = (256, 128, 8), (128, 256, 8) with
// 64 x 64 wave tiles (two waves per SIMD), (128, 256, 4) with 128 x 64
// wave tiles (one wave per SIMD, half the unpack work per MFMA), (64, 512, 8)
// for dense M of 33 to 64 (measured on MI355X at M = 40 to 64: 27-29 us
// against 31-32 us for one partly filled 128-row block, both shapes) and, for
// grouped MoE blocks of 16 rows, (16, 512, 8) with 16 x 64 wave tiles (short
// K: at T = 64, K = 2048, 321 us against 380 us in the streaming family), of
// 32 rows, (32, 512, 8) with 32 x 64 wave tiles (one workgroup per CU with
// three stages; measured on MI355X at E = 256, hidden 7168, T = 512: 7 %
// faster than (32, 256, 4) with two stages and two workgroups per CU), and
// of 64 rows, (64, 512, 8) with 64 x 64 wave tiles and two stages (at
// T = 4096: 11-13 % faster than 128-row blocks, whose padding wastes more
// rows; (64, 256, 4) was slower).
bool tile_cfg_supported(Format f, const TileCfg& c) {
  if (f == FMT_NVFP4 || f == FMT_W8A16 || f == FMT_W2A16) return c.bm == 128 && c.bn == 256 && c.waves == 8;
  if (f != FMT_W4A16) return false;
  if (c.bm == 256 && c.bn == 128) return c.waves == 8;
  if (c.bm == 128 && c.bn == 256) return c.waves == 8 || c.waves == 4;
  if ((c.bm == 16 || c.bm == 32) && c.bn == 512) return c.waves == 8;
  if (c.bm == 64 && c.bn == 512) return c.waves == 8;
  return false;
}

hipError_t launch_tile(Format f, bool asym, bool moe, const TileCfg& c, const GemmArgs& a, int m_blocks,
                       hipStream_t s, KernelLaunch* d) {
  if (!tile_cfg_supported(f, c)) return hipErrorInvalidValue;
  if (f == FMT_NVFP4)
    return moe ? launch_tile_cfg<false, 2, 4, 64, true, true>(a, m_blocks, a.split, s, d)
               : launch_tile_cfg<false, 2, 4, 64, false, true>(a, m_blocks, a.split, s, d);
  if (f == FMT_W8A16)
    return moe ? launch_tile_cfg<false, 2, 4, 64, true, false, true>(a, m_blocks, a.split, s, d)
               : launch_tile_cfg<false, 2, 4, 64, false, false, true>(a, m_blocks, a.split, s, d);
  if (f == FMT_W2A16)
    return moe ? launch_tile_cfg<true, 2, 4, 64, true, false, false, true>(a, m_blocks, a.split, s, d)
               : launch_tile_cfg<true, 2, 4, 64, false, false, false, true>(a, m_blocks, a.split, s, d);
#define QDG_T(ASYM_, WM_, WN_, WTM_, MOE_)                                                 \
  if (asym == ASYM_ && c.bm == WM_ * WTM_ && c.waves == WM_ * WN_ && moe == MOE_)         \
    return launch_tile_cfg<ASYM_, WM_, WN_, WTM_, MOE_>(a, m_blocks, a.split, s, d);
  QDG_T(false, 4, 2, 64, false)
  QDG_T(false, 2, 4, 64, false)
  QDG_T(false, 1, 4, 128, false)
  QDG_T(true, 4, 2, 64, false)
  QDG_T(true, 2, 4, 64, false)
  QDG_T(true, 1, 4, 128, false)
  QDG_T(false, 2, 4, 64, true)
  QDG_T(false, 1, 4, 128, true)
  QDG_T(false, 1, 8, 16, true)
  QDG_T(false, 1, 8, 32, true)
  QDG_T(false, 1, 8, 64, true)
  QDG_T(false, 1, 8, 64, false)
  QDG_T(true, 1, 8, 64, false)
#undef QDG_T
  return hipErrorInvalidValue;
}

hipError_t launch_reduce_splits(const GemmArgs& a, int m_pad, int n_pad, hipStream_t s) {
  const int64_t threads = (int64_t)a.M * (n_pad / 4);
  hipLaunchKernelGGL(reduce_splits_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     (const float*)a.partial, a.Y, a.M, a.N, m_pad, n_pad, a.split, a.otype);
  return hipGetLastError();
}

hipError_t launch_rowsum(const void* a_bf16, const int* sorted_ids, const int* num_padded, int top_k,
                         int a_per_pair, int num_pairs, int M, int K, int m_pad, float factor, float* out,
                         hipStream_t s) {
  const int64_t threads = (int64_t)m_pad * (K / 128) * 16;  // 16 lanes per (row, group)
  hipLaunchKernelGGL(rowsum_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     (const uint16_t*)a_bf16, sorted_ids, num_padded, top_k, a_per_pair, num_pairs, M, K, m_pad,
                     factor, out);
  return hipGetLastError();
}

#endif  // __HIPCC_RTC__

}  // namespace qdg
