// LDS-tiled (large-M) GEMM family for the 8-bit-activation formats:
// W8A8 and W4A8-INT8 (int8 x int8 -> exact int32 on v_mfma_i32_16x16x64_i8)
// and W4A8-MXFP4 (fp8 E4M3 x E2M1 on the scaled 16x16x128 MFMA, with the
// E8M0 block scales applied by the hardware), for W4A4-MXFP4 (E2M1 x E2M1 on
// the same MFMA, both operands' E8M0 scales applied by it) and for MXFP4
// weights x int8 activations (the int8 codes as two exact E4M3 planes, each
// through the fp8 x fp4 MFMA).
//
// The pages' library serves large batches with a different, throughput-
// oriented pipeline than small ones (kinachrichten, "Wie die Architektur
// funktioniert") and names W8A8, W4A8 and the MXFP4 W4A8 path as formats it
// covers ("Warum quantisierte Kernel wichtig sind", "Kompilierzeiten und
// gerätespezifisches Tuning"). The structure is that of the W4A16 LDS-tiled
// family:
//   * a 512-thread workgroup owns a 128 x 256 output tile, its 8 wavefronts
//     (two per SIMD) a 64 x 64 tile each;
//   * the K loop advances one 128-wide group per step; the A tile (128 rows
//     of 128 bytes, padded to 144 so 16-byte fragment reads are conflict-
//     free; fp4: 64 bytes padded to 80), the packed weight units, the
//     per-group weight records and (fp8, fp4) the per-(row, group) activation
//     scales of the next groups are copied
//     global -> LDS by direct LDS loads into a 3-stage ring;
//   * W8A8 accumulates exact int32 over the whole K range and applies the
//     token and channel scales once in the epilogue; W4A8 moves each int4 to
//     the high nibble of an int8 (16 q, exact; 1/16 is folded into the
//     scale), takes an exact int32 partial per group and adds s * P in fp32
//     (raw int32 mode keeps integers throughout); MXFP4 adds a_scale * P per
//     group in fp32; W4A4 accumulates the scaled MFMA results directly;
//   * the output tile goes through LDS so stores are whole 16-byte row
//     segments; split-K writes fp32 partials that reduce_splits_kernel adds
//     in split order;
//   * grouped MoE: each 128-row block of the expert-sorted rows belongs to
//     one expert (moe_align pads every expert's rows to whole blocks), so the
//     workgroup reads that expert's weights once for 128 rows and gathers its
//     A rows (and activation scales) through the sorted row ids; padding rows
//     read row 0 and are never stored.
#ifndef __HIPCC_RTC__
#include <cstdio>
#include <type_traits>
#endif

#include "qdg_device.h"
#include "qdg_internal.h"

namespace qdg {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

enum QKind { Q_W8A8 = 0, Q_W4A8 = 1, Q_MXFP4 = 2, Q_W4A4 = 3, Q_MXFP4_I8 = 4 };

template <int KIND, int BM, int BN>
struct QStage {
  // bytes of A per row and group (MXFP4 x INT8: the hi and lo E4M3 planes)
  static constexpr int AROW = KIND == Q_W4A4 ? 64 : KIND == Q_MXFP4_I8 ? 256 : 128;
  static constexpr int ROW = AROW + 16;                     // + 16 of padding
  static constexpr int CH = ROW / 16;                       // 16-byte slots per row (the last is padding)
  static constexpr int UNIT = KIND == Q_W8A8 ? 2048 : 1024;  // bytes per 16 x 128 weight unit
  static constexpr int A = 0;
  static constexpr int A_SLOTS = BM * ROW / 16;
  static constexpr int AS = BM * ROW;                        // fp8: BM fp32 scales; fp4: BM x 4 E8M0
  static constexpr int W = AS + (KIND == Q_MXFP4 || KIND == Q_W4A4 ? BM * 4 : 0);
  static constexpr int REC = W + (BN / 16) * UNIT;           // W4A8 / MXFP4: 64 bytes per unit
  static constexpr int SCR = REC + (KIND == Q_W8A8 ? 0 : (BN / 16) * 64);  // 1 KiB sink for padding copies
  static constexpr int REC_COPIES = KIND == Q_W8A8 ? 0 : BN / 256;     // 1 KiB record copies per stage
  // at least the 8 waves' 16 x 64 fp32 epilogue strips
  static constexpr int NWAVES = (BM / 64) * (BN / 64);  // 64 x 64 wave tiles
  static constexpr int BYTES = SCR + 1024 > NWAVES * 16 * 64 * 4 ? SCR + 1024 : NWAVES * 16 * 64 * 4;
};

// Copies of group g into stage `st` (device-only builtins: kept out of any
// lambda). A: slot q = 64 i + lane is row q / CH, 16-byte chunk q % CH (the
// last chunk is padding and re-reads chunk 0); a_off holds each slot's row
// offset.
// RAW, MOE and TAG are not used here: they only give every calling function
// its own specialization (hipcc's host pass rejects a second function that
// calls the same specialization of a device function using target builtins):
// TAG = 16 PADSKIP + MT in the K loop, 16 PADSKIP in the kernel's prologue.
template <int KIND, bool RAW, bool MOE, int BM, int BN, int NW, int TAG>
__device__ __forceinline__ void q_load_stage(char* st, const char* a_g, const uint32_t* a_off,
                                             const uint32_t* as_off, const GemmArgs& p, const uint8_t* wbase,
                                             const uint8_t* sbase, int wg_tile0, int wave, int lane, int g) {
  // Every wave issues the same sequence of copies (those past the stage's
  // data re-read a valid address into the sink), without branches: the
  // compiler can then count exactly which copies a later wait covers.
  using L = QStage<KIND, BM, BN>;
  constexpr int A_INST = (L::A_SLOTS + 63) / 64;
  const char* ag = a_g + (size_t)g * L::AROW;
#pragma unroll
  for (int r = 0; r < (A_INST + NW - 1) / NW; ++r) {
    const int i = r * NW + wave;
    const int dst = i < A_INST ? L::A + i * 1024 : L::SCR;
    __builtin_amdgcn_global_load_lds(ag + a_off[r], (lds_void*)(st + dst), 16, 0, 0);
  }
  constexpr int W_INST = (BN / 16) * (L::UNIT / 1024);
#pragma unroll
  for (int r = 0; r < (W_INST + NW - 1) / NW; ++r) {
    const int i = min(r * NW + wave, W_INST - 1);
    const int dst = r * NW + wave < W_INST ? L::W + i * 1024 : L::SCR;
    const int t = i / (L::UNIT / 1024), h = i % (L::UNIT / 1024);
    // tiles past the layer re-read the last tile; their results are never stored
    const int tile = min(wg_tile0 + t, p.ntiles - 1);
    __builtin_amdgcn_global_load_lds(wbase + ((size_t)tile * p.groups + g) * L::UNIT + h * 1024 + lane * 16,
                                     (lds_void*)(st + dst), 16, 0, 0);
  }
  // records: copy r (16 tiles of 64 bytes) by wave NW - 1 - r; every wave
  // issues REC_COPIES copies, the others into the sink
#pragma unroll
  for (int r = 0; r < L::REC_COPIES; ++r) {
    const int tile = min(wg_tile0 + 16 * r + (lane >> 2), p.ntiles - 1);
    __builtin_amdgcn_global_load_lds(sbase + ((size_t)tile * p.groups + g) * 64 + (lane & 3) * 16,
                                     (lds_void*)(st + (wave == NW - 1 - r ? L::REC + r * 1024 : L::SCR)), 16, 0, 0);
  }
  if constexpr (KIND == Q_MXFP4 || KIND == Q_W4A4) {
    // activation scales a_scales[row][g] (fp8: one fp32; fp4: the 4 E8M0
    // bytes of the group's 32-blocks), one dword per row
#pragma unroll
    for (int r = 0; r < BM / 64; ++r)
      __builtin_amdgcn_global_load_lds((const char*)p.a_scales + as_off[r] + (size_t)g * 4,
                                       (lds_void*)(st + (wave == r % NW ? L::AS + r * 256 : L::SCR)), 4, 0, 0);
  }
}

// The LDS fragments one wave needs for one K group of its 64 x 64 tile
// (4 x 4 MFMA tiles of 16 x 16).
template <int KIND>
struct QFrag {
  u32x4_t a[4][KIND == Q_MXFP4_I8 ? 4 : 2];  // A rows of the 4 row tiles (16-byte K slices; I8: hi, then lo)
  u32x4_t b[4][2];  // weights of the 4 column tiles (W4A8: packed int4 in b[t][0])
  float ws[4];      // W4A8: group scale s/16 of the lane's column
  int e8[4];        // MXFP4, W4A4: E8M0 block scale of the lane
  f32x4_t as[4];    // MXFP4: activation scales of the lane's 4 rows
  int ae8[4];       // W4A4: E8M0 scale of the lane's A row and 32-block
};

// MT: the row tiles read and multiplied (2: the wave's rows 32..63 are
// padding of a grouped MoE block)
template <int KIND, int BM, int BN, int MT = 4>
__device__ __forceinline__ void q_frag_load(QFrag<KIND>& f, const char* st, int a_lane, int w_lane, int rec_lane,
                                            int as_lane) {
  using L = QStage<KIND, BM, BN>;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if constexpr (KIND == Q_W8A8) {
      f.b[t][0] = *(const u32x4_t*)(st + w_lane + t * 2048);
      f.b[t][1] = *(const u32x4_t*)(st + w_lane + t * 2048 + 1024);
    } else {
      f.b[t][0] = *(const u32x4_t*)(st + w_lane + t * 1024);
      if constexpr (KIND == Q_W4A8)
        f.ws[t] = *(const float*)(st + rec_lane + t * 64);
      else
        f.e8[t] = *(const uint8_t*)(st + rec_lane + t * 64);
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    // int8 operand: lane group c holds K 32c..32c+15 (step 0) and +16 (step 1);
    // fp8 operand: K 16c..16c+15 and 64+16c..64+16c+15
    // fp4 operand: K 32c..32c+31 (16 bytes)
    f.a[mt][0] = *(const u32x4_t*)(st + a_lane + mt * 16 * L::ROW);
    if constexpr (KIND != Q_W4A4)
      f.a[mt][1] = *(const u32x4_t*)(st + a_lane + mt * 16 * L::ROW + (KIND == Q_MXFP4 || KIND == Q_MXFP4_I8 ? 64 : 16));
    if constexpr (KIND == Q_MXFP4_I8) {  // the lo plane, 128 bytes on
      f.a[mt][2] = *(const u32x4_t*)(st + a_lane + mt * 16 * L::ROW + 128);
      f.a[mt][3] = *(const u32x4_t*)(st + a_lane + mt * 16 * L::ROW + 192);
    }
    if constexpr (KIND == Q_MXFP4) f.as[mt] = *(const f32x4_t*)(st + as_lane + mt * 64);
    if constexpr (KIND == Q_W4A4) f.ae8[mt] = *(const uint8_t*)(st + as_lane + mt * 64);
  }
}

template <int KIND, bool RAW, bool MOE, int BM, int MT, class Acc>  // MOE, BM: a specialization per kernel, as above
__device__ __forceinline__ void q_frag_compute(const QFrag<KIND>& f, Acc (&acc)[4][4]) {
  u32x4_t b[4][2];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if constexpr (KIND == Q_W4A8) {
      const u32x4_t x = f.b[t][0];
      const u32x2_t l0 = unpack_i4_i8x16(x.x), h0 = unpack_i4_i8x16(x.y);
      const u32x2_t l1 = unpack_i4_i8x16(x.z), h1 = unpack_i4_i8x16(x.w);
      b[t][0] = u32x4_t{l0.x, l0.y, h0.x, h0.y};
      b[t][1] = u32x4_t{l1.x, l1.y, h1.x, h1.y};
    } else {
      b[t][0] = f.b[t][0];
      b[t][1] = f.b[t][1];
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if constexpr (KIND == Q_W4A4) {
        const u32x4_t a0 = f.a[mt][0];
        const i32x8_t av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, 0, 0, 0, 0};
        const i32x8_t bv = {(int)b[t][0].x, (int)b[t][0].y, (int)b[t][0].z, (int)b[t][0].w, 0, 0, 0, 0};
        acc[mt][t] = mfma_fp4_fp4_scaled(av, bv, acc[mt][t], f.ae8[mt], f.e8[t]);
      } else if constexpr (KIND == Q_MXFP4_I8) {
        // int8 = 16 hi + lo, both exact in E4M3: the hi plane with A scale
        // 2^4 (E8M0 131), the lo plane with 2^0, the weights' E8M0 on both;
        // the products are exact and accumulate over the whole K range (the
        // token scale is applied once in the epilogue)
        const u32x4_t h0 = f.a[mt][0], h1 = f.a[mt][1], l0 = f.a[mt][2], l1 = f.a[mt][3];
        const i32x8_t ah = {(int)h0.x, (int)h0.y, (int)h0.z, (int)h0.w, (int)h1.x, (int)h1.y, (int)h1.z, (int)h1.w};
        const i32x8_t al = {(int)l0.x, (int)l0.y, (int)l0.z, (int)l0.w, (int)l1.x, (int)l1.y, (int)l1.z, (int)l1.w};
        const i32x8_t bv = {(int)b[t][0].x, (int)b[t][0].y, (int)b[t][0].z, (int)b[t][0].w, 0, 0, 0, 0};
        acc[mt][t] = mfma_fp8_fp4_scaled(al, bv, mfma_fp8_fp4_scaled(ah, bv, acc[mt][t], 131, f.e8[t]), 127, f.e8[t]);
      } else if constexpr (KIND == Q_MXFP4) {
        const u32x4_t a0 = f.a[mt][0], a1 = f.a[mt][1];
        const i32x8_t av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        const i32x8_t bv = {(int)b[t][0].x, (int)b[t][0].y, (int)b[t][0].z, (int)b[t][0].w, 0, 0, 0, 0};
        const f32x4_t pr = mfma_fp8_fp4_scaled(av, bv, f32x4_t{0.f, 0.f, 0.f, 0.f}, 127, f.e8[t]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mt][t][i] = __builtin_fmaf(f.as[mt][i], pr[i], acc[mt][t][i]);
      } else if constexpr (KIND == Q_W8A8 || RAW) {
        acc[mt][t] = mfma_i8(f.a[mt][1], b[t][1], mfma_i8(f.a[mt][0], b[t][0], acc[mt][t]));
      } else {
        const i32x4_t pr = mfma_i8(f.a[mt][1], b[t][1], mfma_i8(f.a[mt][0], b[t][0], i32x4_t{0, 0, 0, 0}));
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mt][t][i] = __builtin_fmaf(f.ws[t], (float)pr[i], acc[mt][t][i]);
      }
    }
  }
}

template <int KIND, bool RAW>
struct QAcc {
  using T = typename std::conditional<KIND == Q_W8A8 || RAW, i32x4_t, f32x4_t>::type;
};

// The K loop of the 8-bit tile over groups [g0, g1) (the first NS - 1
// stages already in flight): full rounds of NS groups run unrolled with
// constant stage indices; MT row tiles of the wave are read and multiplied.
template <int KIND, bool RAW, int NS, bool MOE, int BM, int BN, int NW, int VM_NEXT, bool PADSKIP, int MT, class Acc>
__device__ __forceinline__ void q_k_loop(char* const (&stage)[3], const char* a_g, const uint32_t* a_off,
                                         const uint32_t* as_off, const GemmArgs& p, const uint8_t* wbase,
                                         const uint8_t* sbase, int wg_tile0, int wave, int lane, int g0, int g1,
                                         int a_lane, int w_lane, int rec_lane, int as_lane, Acc (&acc)[4][4]) {
  QFrag<KIND> fr;
  int gb = g0;
  for (; gb + NS <= g1; gb += NS) {
#pragma unroll
    for (int cur = 0; cur < NS; ++cur) {
      // this wave's copies of group gb+cur are done once at most the copies
      // of the NS - 2 later groups in flight remain (copies complete in
      // order; with two stages nothing later is in flight yet)
      constexpr int VM_LEFT = VM_NEXT * (NS - 2);
      __builtin_amdgcn_s_waitcnt((VM_LEFT & 15) | (7 << 4) | (15 << 8) | ((VM_LEFT >> 4) << 14));
      // every wave's copies of the group landed; the stage of the previous
      // group is free. A bare s_barrier: __syncthreads would also wait for
      // the copies in flight.
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      asm volatile("s_barrier" ::: "memory");
      q_load_stage<KIND, RAW, MOE, BM, BN, NW, 16 * PADSKIP + MT>(stage[(cur + NS - 1) % NS], a_g, a_off, as_off, p,
                                                                 wbase, sbase, wg_tile0, wave, lane,
                                                                 min(gb + cur + NS - 1, g1 - 1));
      q_frag_load<KIND, BM, BN, MT>(fr, stage[cur], a_lane, w_lane, rec_lane, as_lane);
      // MXFP4: all of the group's fragment reads go out before its first
      // MFMA (left to itself the scheduler sinks each row tile's reads next
      // to its MFMAs, and every row tile then waits out a full LDS latency;
      // measured on MI355X at M = 4096: 84 -> 78 us at K = 7168, 113 -> 110 us
      // at K = 2048; the int8 formats run as fast or faster without it)
      if constexpr (KIND == Q_MXFP4) __builtin_amdgcn_sched_barrier(0);
      q_frag_compute<KIND, RAW, MOE, BM, MT>(fr, acc);
    }
  }
#pragma unroll
  for (int cur = 0; cur < NS - 1; ++cur) {
    if (gb + cur < g1) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      q_frag_load<KIND, BM, BN, MT>(fr, stage[cur], a_lane, w_lane, rec_lane, as_lane);
      q_frag_compute<KIND, RAW, MOE, BM, MT>(fr, acc);
    }
  }
}

// PADSKIP (grouped MoE): a wave whose rows 32..63 are all padding runs a
// second instance of the K loop without their fragment reads and MFMAs (an
// expert's real entries lead its blocks, so the entry at row 32 tells). Both
// instances run the same barriers, so the waves of one workgroup may take
// different ones. It is a separate kernel instance because the second K loop
// changes how the compiler schedules the first (every copy of a group issued
// right after the barrier), which measured slower where most blocks are full.
template <int KIND, bool RAW, int NS, bool MOE, int WAVES_M = 2, int WAVES_N = 4, bool PADSKIP = false>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void qtile_gemm_kernel(const GemmArgs p, int m_blocks,
                                                                            int n_blocks) {
  constexpr int NW = WAVES_M * WAVES_N, WTM = 64;
  constexpr int BM = WTM * WAVES_M, BN = 64 * WAVES_N;
  using L = QStage<KIND, BM, BN>;
  using Acc = typename QAcc<KIND, RAW>::T;
  constexpr int A_INST = (L::A_SLOTS + 63) / 64;
  constexpr int A_PER_WAVE = (A_INST + NW - 1) / NW;
  constexpr int W_INST = (BN / 16) * (L::UNIT / 1024);
  // copies every wave issues per stage; waiting for the count to drop to
  // this leaves the next stage in flight
  constexpr int VM_NEXT = (A_INST + NW - 1) / NW + (W_INST + NW - 1) / NW + L::REC_COPIES +
                          (KIND == Q_MXFP4 || KIND == Q_W4A4 ? BM / 64 : 0);
  static_assert(NS == 2 || NS == 3, "two or three stages");
  static_assert(VM_NEXT * (NS - 2) < 64, "vmcnt holds the copies in flight");
  // The stages are separate LDS objects (not one dynamic array) so that the
  // compiler can tell a copy into one stage from a read of another: reads of
  // stage s then wait only for the copies of stage s.
  __shared__ __attribute__((aligned(1024))) char st0[L::BYTES];
  __shared__ __attribute__((aligned(1024))) char st1[L::BYTES];
  __shared__ __attribute__((aligned(1024))) char st2[NS == 3 ? L::BYTES : 16];
  char* const stage[3] = {st0, st1, st2};

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int c = lane >> 4, col = lane & 15;

  // XCD-aware tile order: consecutive workgroup ids go to different XCDs,
  // so XCD x takes the x-th eighth of the tile order; that order walks 4 x 8
  // blocks of tiles, so the 32 tiles an XCD runs at once share 4 row blocks
  // of A and 8 column blocks of W in its L2 (grouped MoE: moe_tile_order)
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
  const int split = blockIdx.y, nsplit = gridDim.y;
  const int g0 = (int)(((int64_t)split * p.groups) / nsplit);
  const int g1 = (int)(((int64_t)(split + 1) * p.groups) / nsplit);

  int expert = 0;
  if constexpr (MOE) {
    if (mb * BM >= *p.num_padded) return;  // the whole workgroup leaves together
    expert = p.block_expert[mb];
  }
  const uint8_t* wbase = p.packed + (size_t)expert * p.expert_stride;
  const uint8_t* sbase = wbase + p.s_offset;
  const int wg_tile0 = nb * (BN / 16);
  // the A row (and activation-scale row) behind output row `grow` of the
  // tile, and whether that row is stored
  auto a_row = [&](int grow) -> int {
    if constexpr (MOE) {
      const int id = p.sorted_ids[grow];
      return id < p.num_pairs ? (p.a_per_pair ? id : id / p.top_k) : 0;
    } else {
      return grow < p.M ? grow : p.M - 1;
    }
  };

  uint32_t a_off[A_PER_WAVE];
#pragma unroll
  for (int r = 0; r < A_PER_WAVE; ++r) {
    const int q = (r * NW + wave) * 64 + lane;
    const int row = min(q / L::CH, BM - 1), ch = q % L::CH;
    const int src = a_row(mb * BM + row);
    const uint32_t a_bytes = KIND == Q_W4A4 ? (uint32_t)p.K / 2 : KIND == Q_MXFP4_I8 ? 2u * p.K : (uint32_t)p.K;
    a_off[r] = (uint32_t)src * a_bytes + (uint32_t)(ch < L::CH - 1 ? ch : 0) * 16;
  }
  uint32_t as_off[BM / 64];
#pragma unroll
  for (int r = 0; r < BM / 64; ++r) {
    const int src = a_row(mb * BM + r * 64 + lane);
    as_off[r] = (uint32_t)src * (uint32_t)p.groups * 4u;
  }

  // per-lane LDS offsets of the fragment reads inside a stage
  const int a_lane =
      L::A + (wm * WTM + col) * L::ROW + (KIND == Q_MXFP4 || KIND == Q_W4A4 || KIND == Q_MXFP4_I8 ? 16 : 32) * c;
  const int w_lane = L::W + (wn * 4) * L::UNIT + lane * 16;
  const int rec_lane =
      L::REC + (wn * 4) * 64 + (KIND == Q_MXFP4 || KIND == Q_W4A4 || KIND == Q_MXFP4_I8 ? lane : col * 4);
  // fp8: the fp32 scales of the lane's 4 D rows; fp4: the E8M0 byte of the
  // lane's A row and 32-block
  const int as_lane = KIND == Q_W4A4 ? L::AS + (wm * WTM + col) * 4 + c : L::AS + (wm * WTM + 4 * c) * 4;

  Acc acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[mt][t] = Acc{0, 0, 0, 0};

  const char* a_g = (const char*)p.A;
  // NS-stage ring. Full rounds of NS groups run unrolled with constant stage
  // indices and unconditional copies (past the range they re-read the last
  // group into a stage nobody reads again), so that the compiler's waits
  // before LDS reads stay exact; the last partial round waits for all copies.
#pragma unroll
  for (int q = 0; q < NS - 1; ++q)
    q_load_stage<KIND, RAW, MOE, BM, BN, NW, 16 * PADSKIP>(stage[q], a_g, a_off, as_off, p, wbase, sbase, wg_tile0,
                                                          wave, lane, min(g0 + q, g1 - 1));
  if constexpr (PADSKIP) {
    static_assert(MOE, "padding halves exist in grouped MoE blocks only");
    if (p.sorted_ids[mb * BM + wm * WTM + 32] >= p.num_pairs)
      q_k_loop<KIND, RAW, NS, MOE, BM, BN, NW, VM_NEXT, PADSKIP, 2>(
          stage, a_g, a_off, as_off, p, wbase, sbase, wg_tile0, wave, lane, g0, g1, a_lane, w_lane, rec_lane,
          as_lane, acc);
    else
      q_k_loop<KIND, RAW, NS, MOE, BM, BN, NW, VM_NEXT, PADSKIP, 4>(
          stage, a_g, a_off, as_off, p, wbase, sbase, wg_tile0, wave, lane, g0, g1, a_lane, w_lane, rec_lane,
          as_lane, acc);
  } else {
    q_k_loop<KIND, RAW, NS, MOE, BM, BN, NW, VM_NEXT, PADSKIP, 4>(
        stage, a_g, a_off, as_off, p, wbase, sbase, wg_tile0, wave, lane, g0, g1, a_lane, w_lane, rec_lane,
        as_lane, acc);
  }

  // ---- epilogue: scale, then per wave transpose each 16 x 64 strip through
  // LDS so that every lane stores whole 16-byte row segments
  __builtin_amdgcn_s_waitcnt(0);  // the trailing copies have landed
  __syncthreads();
  const bool to_partial = nsplit > 1;
  const int n_pad = n_blocks * BN;
  const bool raw = p.otype == QDG_O_I32;
  const bool f32out = to_partial || p.otype == QDG_O_F32 || raw;  // 4-byte elements
  char* strip = st0 + wave * (16 * 64 * 4);
  static_assert(NW * 16 * 64 * 4 <= L::BYTES, "epilogue strips fit one stage");
  const int nbase = (wg_tile0 + wn * 4) * 16;
  const int esz = f32out ? 4 : 2;
  const int cpr = 64 * esz / 16;  // 16-byte chunks per strip row
  float wsc[4] = {1.f, 1.f, 1.f, 1.f};
  if constexpr (KIND == Q_W8A8) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int tile = min(wg_tile0 + wn * 4 + t, p.ntiles - 1);
      wsc[t] = ((const float*)sbase)[tile * 16 + col];
    }
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    float asc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int grow = mb * BM + wm * WTM + mt * 16 + 4 * c + i;
      asc[i] = (KIND != Q_MXFP4 && KIND != Q_W4A4 && !raw && (MOE || grow < p.M)) ? p.a_scales[a_row(grow)] : 1.f;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = (4 * c + i) * 64 + t * 16 + col;
        uint32_t bits;
        if (raw) {
          int v = bits_as<int>(acc[mt][t][i]);
          if constexpr (KIND == Q_W4A8) v >>= 4;  // 16 q * qa: exact shift back
          bits = (uint32_t)v;
        } else {
          float y;
          if constexpr (KIND == Q_W8A8)
            y = (float)acc[mt][t][i] * asc[i] * wsc[t];
          else if constexpr (KIND == Q_W4A8 || KIND == Q_MXFP4_I8)
            y = acc[mt][t][i] * asc[i];
          else
            y = acc[mt][t][i];
          bits = f32out ? __builtin_bit_cast(uint32_t, y) : f32_to_bf16_rne(y);
        }
        if (f32out)
          ((uint32_t*)strip)[e] = bits;
        else
          ((uint16_t*)strip)[e] = (uint16_t)bits;
      }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    for (int chunk = lane; chunk < 16 * cpr; chunk += 64) {
      const int r = chunk / cpr, cc = chunk % cpr;
      const int lrow = mb * BM + wm * WTM + mt * 16 + r;
      int yrow = lrow;
      bool v;
      if constexpr (MOE) {
        yrow = p.sorted_ids[lrow];
        v = yrow < p.num_pairs;
      } else {
        v = lrow < p.M;
      }
      const int per = 16 / esz;  // elements per chunk
      const int n0 = nbase + cc * per;
      const u32x4_t val = *(const u32x4_t*)(strip + r * 64 * esz + cc * 16);
      if (to_partial) {
        *(u32x4_t*)((float*)p.partial + ((size_t)split * p.m_pad + lrow) * n_pad + n0) = val;
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
// One launch of qtile_gemm_kernel<KIND, RAW, NS, MOE, WM, WN>, or its
// description (desc set).
template <int KIND, bool RAW, int NS, bool MOE, int WM, int WN, bool PADSKIP = false>
hipError_t launch_q_inst(const GemmArgs& a, dim3 grid, int m_blocks, int n_blocks, hipStream_t s, KernelLaunch* d) {
  if (d) {
    d->src = JIT_SRC_QTILE;
    std::snprintf(d->expr, sizeof d->expr, "qdg::qtile_gemm_kernel<%d, %s, %d, %s, %d, %d, %s>", KIND,
                  RAW ? "true" : "false", NS, MOE ? "true" : "false", WM, WN, PADSKIP ? "true" : "false");
    d->grid[0] = grid.x;
    d->grid[1] = grid.y;
    d->grid[2] = 1;
    d->block = 64 * WM * WN;
    d->mn_args = true;
    d->m_blocks = m_blocks;
    d->n_blocks = n_blocks;
    return hipSuccess;
  }
  hipLaunchKernelGGL((qtile_gemm_kernel<KIND, RAW, NS, MOE, WM, WN, PADSKIP>), grid, dim3(64 * WM * WN), 0, s, a,
                     m_blocks, n_blocks);
  return hipGetLastError();
}

template <int KIND, bool RAW>
hipError_t launch_q(const GemmArgs& a, bool moe, int bm, int m_blocks, int nsplit, bool pad_skip, hipStream_t s,
                    KernelLaunch* d) {
  if (moe && nsplit != 1) return hipErrorInvalidValue;  // grouped MoE is not split
  if (moe && bm == 64) {
    // 64-row expert blocks: 64 x 512 tiles, 8 waves in one row
    constexpr int BM = 64, BN = 512;
    constexpr int NS = 3 * QStage<KIND, BM, BN>::BYTES <= 160 * 1024 ? 3 : 2;
    const int n_blocks = (a.ntiles + BN / 16 - 1) / (BN / 16);
    const dim3 grid(moe_grid_blocks(m_blocks) * n_blocks, 1);
    return pad_skip ? launch_q_inst<KIND, RAW, NS, true, 1, 8, true>(a, grid, m_blocks, n_blocks, s, d)
                    : launch_q_inst<KIND, RAW, NS, true, 1, 8>(a, grid, m_blocks, n_blocks, s, d);
  }
  if (bm != 128) return hipErrorInvalidValue;
  constexpr int BM = 128, BN = 256;
  using L = QStage<KIND, BM, BN>;
  constexpr int NS = 3 * L::BYTES <= 160 * 1024 ? 3 : 2;
  const int n_blocks = (a.ntiles + BN / 16 - 1) / (BN / 16);
  if (moe) {
    const dim3 grid(moe_grid_blocks(m_blocks) * n_blocks, 1);
    return pad_skip ? launch_q_inst<KIND, RAW, NS, true, 2, 4, true>(a, grid, m_blocks, n_blocks, s, d)
                    : launch_q_inst<KIND, RAW, NS, true, 2, 4>(a, grid, m_blocks, n_blocks, s, d);
  }
  return launch_q_inst<KIND, RAW, NS, false, 2, 4>(a, dim3(m_blocks * n_blocks, nsplit), m_blocks, n_blocks, s, d);
}
#endif  // __HIPCC_RTC__

}  // namespace

#ifndef __HIPCC_RTC__  // host launchers
hipError_t launch_qtile(Format f, bool moe, int bm, bool pad_skip, const GemmArgs& a, int m_blocks, hipStream_t s,
                        KernelLaunch* d) {
  const bool raw = a.otype == QDG_O_I32;
  if (raw && a.split > 1) return hipErrorInvalidValue;  // integer partials are not split
  switch (f) {
    case FMT_W8A8:
      return raw ? launch_q<Q_W8A8, true>(a, moe, bm, m_blocks, 1, pad_skip, s, d)
                 : launch_q<Q_W8A8, false>(a, moe, bm, m_blocks, a.split, pad_skip, s, d);
    case FMT_W4A8:
      return raw ? launch_q<Q_W4A8, true>(a, moe, bm, m_blocks, 1, pad_skip, s, d)
                 : launch_q<Q_W4A8, false>(a, moe, bm, m_blocks, a.split, pad_skip, s, d);
    case FMT_MXFP4: return launch_q<Q_MXFP4, false>(a, moe, bm, m_blocks, a.split, pad_skip, s, d);
    case FMT_W4A4: return launch_q<Q_W4A4, false>(a, moe, bm, m_blocks, a.split, pad_skip, s, d);
    case FMT_MXFP4_I8: return launch_q<Q_MXFP4_I8, false>(a, moe, bm, m_blocks, a.split, pad_skip, s, d);
    default: return hipErrorInvalidValue;
  }
}

#endif  // __HIPCC_RTC__

}  // namespace qdg
