// Weight-streaming W4A16 kernel for M <= 16 (dense) and for the grouped MoE
// GEMM when an expert block holds 16 rows.
//
// At this size the layer is a stream of packed weights from HBM and the
// kernel's job is to keep enough of that stream in flight on every CU while
// the small MFMA work hides under it:
//   * a workgroup of 8 waves owns 4 adjacent 16-column N tiles and a K range;
//     wave w works on tile w % 4 and on half w / 4 of every 16-group chunk;
//   * chunks are software-pipelined: while chunk i is computed, the 8 weight
//     units of chunk i+1 of every wave, that chunk's A rows (only the M rows
//     that exist; wave w stages rows 2w and 2w+1) and its scale records are
//     in flight into registers; at the top of chunk i+1 the A rows go to the
//     other half of a double-buffered LDS area, shared by the 8 waves;
//   * every global load has a register destination, so the compiler's load
//     waits are exact and the next chunk's loads stay in flight through the
//     current chunk's compute (copies straight into LDS would make it wait
//     for all of them before any LDS read);
//   * the MFMA chains of a group start from -(128+z) * rowsum(A) (the
//     streaming family's offset trick); the row sums of a chunk are computed
//     once per workgroup, two groups per wave, by MFMAs against a constant;
//   * the two K halves are added through LDS in a fixed order; when the N
//     tiles cannot occupy the CUs (4096-wide down projections) K is also
//     split across workgroups and reduce_splits_kernel adds the fp32
//     partials in split order (deterministic, no device-scope fences).
// The pages' small-batch design streams weights through a multi-stage
// asynchronous copy pipeline (kinachrichten, "Wie die Architektur
// funktioniert"); a register-level pipeline with double-buffered LDS A
// chunks is the gfx950 form of that idea.
#ifndef __HIPCC_RTC__
#include <cstdio>
#endif

#include "qdg_device.h"
#include "qdg_internal.h"

namespace qdg {
namespace {

constexpr int NT = 4;                      // N tiles per workgroup
constexpr int KW = 2;                      // K halves per chunk
constexpr int WAVES = NT * KW;             // 8
constexpr int CG = 4;                      // groups per wave per chunk
constexpr int CGW = KW * CG;               // 8 groups per chunk
constexpr int A_PITCH = CGW * 256 + 16;    // 2064-byte LDS rows: conflict-free fragment reads
constexpr int A_BYTES = 16 * A_PITCH;
constexpr int AL = CGW * 256 / 1024;       // 16-byte loads per lane per A row (2)
constexpr int S_BYTES = WAVES * CG * 128;  // each wave's CG groups of 16 records
constexpr int C_BYTES = CGW * 16 * 4;      // row sums of the chunk
constexpr int BUF = A_BYTES + S_BYTES + C_BYTES;
static_assert(2 * BUF <= 160 * 1024, "fits the LDS of one CU");
static_assert(NT * 16 * 16 * 4 <= BUF, "K-half exchange fits one buffer");
static_assert(WAVES * 2 == 16, "two A rows per wave");
static_assert(CGW % WAVES == 0 && AL >= 1, "row sums: whole groups per wave");
static_assert(CG * 8 <= 64, "one record load per wave and chunk");

__shared__ __attribute__((aligned(1024))) char ws_lds0[BUF];
__shared__ __attribute__((aligned(1024))) char ws_lds1[BUF];

template <int B>
__device__ __forceinline__ char* ws_buf() {
  return B ? ws_lds1 : ws_lds0;
}

// Workgroup barrier for LDS data: this wave's LDS writes complete, then
// s_barrier (global loads in flight are left alone).
__device__ __forceinline__ void ws_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt untouched
  asm volatile("s_barrier" ::: "memory");
}

struct WsCtx {
  const char* arow[2];  // this wave's two A rows (+ lane * 16)
  const uint8_t* wt;    // this wave's tile: weight units of group 0, + lane * 16
  const uint8_t* srec;  // this wave's tile: records of group 0
  int g0, g1, kp, wave, lane, nchunks;
  bool stage_a;         // this wave has a row that exists
};

// Registers in flight for one chunk.
struct WsChunkRegs {
  u32x4_t a[2][AL];  // A rows 2w, 2w+1 of the chunk
  u32x4_t s;         // scale records: group l / 8, bytes 16 (l % 8)
  u32x4_t w[CG];     // weight units
};

// Issue every load of the chunk at group gbase (clamped to the last chunk).
// Slots past the chunk's groups re-read the chunk's first slot, units and
// records past the range re-read the last valid ones: a fixed count of
// in-bounds loads on every path.
__device__ __forceinline__ void ws_issue(WsChunkRegs& r, const WsCtx& x, int gbase) {
  const int gsz = min(CGW, x.g1 - gbase);
  // records: lane l holds group l / 8, bytes 16 (l % 8); lanes past the
  // wave's CG groups re-read its last group (only the first CG * 8 are kept)
  int g = gbase + x.kp * CG + min(x.lane >> 3, CG - 1);
  g = g < x.g1 ? g : x.g1 - 1;
  r.s = *(const u32x4_t*)(x.srec + (size_t)g * 128 + (x.lane & 7) * 16);
  if (x.stage_a) {  // wave-uniform
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int k = 0; k < AL; ++k) {
        const int slot = k * 64 + x.lane;  // 16-byte slot of the chunk row
        const int sl = slot < gsz * 16 ? slot : 0;
        r.a[h][k] = *(const u32x4_t*)(x.arow[h] + (size_t)gbase * 256 + sl * 16 - x.lane * 16);
      }
  }
  const int first = gbase + x.kp * CG;
#pragma unroll
  for (int u = 0; u < CG; ++u) {
    const int gu = first + u < x.g1 ? first + u : x.g1 - 1;
    r.w[u] = ldg_nt((const u32x4_t*)(x.wt + (size_t)gu * kUnit4Bytes));
  }
}

// One pipelined chunk: stage chunk i's A rows and records, start chunk i+1
// (unless this is the last chunk, PF = false), compute chunk i.
template <bool ASYM, int B, bool PF>
__device__ __forceinline__ void ws_chunk(const WsCtx& x, int i, WsChunkRegs& cur, WsChunkRegs& nxt, f32x4_t& acc,
                                         uint32_t um, uint32_t ue) {
  const int lane = x.lane, c = lane >> 4, col = lane & 15;
  char* buf = ws_buf<B>();
  const int gbase = x.g0 + i * CGW;
  const int gsz = min(CGW, x.g1 - gbase);
  // buffer B was last read in chunk i-2, which every wave finished before
  // the barriers of chunk i-1
  if (x.stage_a) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int k = 0; k < AL; ++k)
        *(u32x4_t*)(buf + (2 * x.wave + h) * A_PITCH + (k * 64 + lane) * 16) = cur.a[h][k];
  }
  if (lane < CG * 8) *(u32x4_t*)(buf + A_BYTES + x.wave * (CG * 128) + lane * 16) = cur.s;
  ws_barrier();
  if constexpr (PF) ws_issue(nxt, x, gbase + CGW);
  // Row sums of the chunk's groups (pre-scaled by -136 when symmetric). All
  // 16 groups and all 8 units of a wave are computed without branches, so
  // that the compiler's load waits stay exact (they count the loads issued
  // after the one waited for on every path); groups past the range (their
  // data are in-bounds re-reads, finite) are dropped by a select.
  float* corr = (float*)(buf + A_BYTES + S_BYTES);
#pragma unroll
  for (int h = 0; h < CGW / WAVES; ++h) {
    const int q = x.wave + h * WAVES;
    f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    const u32x4_t kb = ASYM ? u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u}   // bf16 1.0
                            : u32x4_t{0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u};  // bf16 -136
#pragma unroll
    for (int j = 0; j < 4; ++j)
      z = mfma_bf16(*(const u32x4_t*)(buf + col * A_PITCH + q * 256 + (4 * c + j) * 16), kb, z);
    if (col == 0) *(f32x4_t*)(corr + q * 16 + 4 * c) = z;
  }
  ws_barrier();
  const char* srecs = buf + A_BYTES + x.wave * (CG * 128);
#pragma unroll
  for (int u = 0; u < CG; ++u) {
    const int q = x.kp * CG + u;
    u32x4_t a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = *(const u32x4_t*)(buf + col * A_PITCH + q * 256 + (4 * c + j) * 16);
    const f32x4_t rs = *(const f32x4_t*)(corr + q * 16 + 4 * c);
    const u32x2_t rec = *(const u32x2_t*)(srecs + u * 128 + col * 8);
    f32x4_t pacc;
    if constexpr (ASYM) {
      const float negz = __builtin_bit_cast(float, (rec.y & 0xFFFFu) << 16);  // -(128+z)
      pacc = f32x4_t{negz * rs[0], negz * rs[1], negz * rs[2], negz * rs[3]};
    } else {
      pacc = rs;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) pacc = mfma_bf16(a[j], unpack_u4_bf16_offset128(cur.w[u][j], um, ue), pacc);
    const float s = bits_as<float>(rec.x);
    const bool valid = q < gsz;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = valid ? __builtin_fmaf(s, pacc[e], acc[e]) : acc[e];
  }
}

// Output of one 16x16 tile: lane holds rows 4c+e of column `col`; with a K
// split the fp32 partial goes to [split][16][n_pad] in the workspace.
template <bool MOE>
__device__ __forceinline__ void ws_store(const GemmArgs& p, const f32x4_t& acc, int tile, int split, int mb, int c,
                                         int col) {
  const int n = tile * 16 + col;
  if (gridDim.y > 1) {
    const int n_pad = p.ntiles * 16;
#pragma unroll
    for (int e = 0; e < 4; ++e) ((float*)p.partial)[((size_t)split * 16 + 4 * c + e) * n_pad + n] = acc[e];
    return;
  }
  if (n >= p.N) return;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = 4 * c + e;
    int yrow = r;
    bool v;
    if constexpr (MOE) {
      const int id = p.sorted_ids[mb * 16 + r];
      v = id < p.num_pairs;
      yrow = id;
    } else {
      v = r < p.M;
    }
    if (!v) continue;
    const size_t o = (size_t)yrow * p.N + n;
    if (p.otype == QDG_O_F32)
      ((float*)p.Y)[o] = acc[e];
    else
      ((uint16_t*)p.Y)[o] = (uint16_t)f32_to_bf16_rne(acc[e]);
  }
}

template <bool ASYM, bool MOE>
__global__ __launch_bounds__(512) void wstream_kernel(const GemmArgs p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane >> 4, col = lane & 15;
  const int t = wave % NT, kp = wave / NT;
  const int nb = blockIdx.x, split = blockIdx.y, mb = blockIdx.z;

  int expert = 0;
  if constexpr (MOE) {
    if (mb * 16 >= *p.num_padded) return;
    expert = p.block_expert[mb];
  }
  const uint8_t* wbase = p.packed + (size_t)expert * p.expert_stride;
  const int groups = p.groups;
  const int tile = nb * NT + t;
  const int ltile = tile < p.ntiles ? tile : p.ntiles - 1;  // clamped (never stored)

  WsCtx x;
  x.wt = wbase + (size_t)ltile * groups * kUnit4Bytes + lane * 16;
  x.srec = wbase + p.s_offset + (size_t)ltile * groups * 128;
  x.g0 = (int)(((int64_t)split * groups) / gridDim.y);
  x.g1 = (int)(((int64_t)(split + 1) * groups) / gridDim.y);
  x.kp = kp;
  x.wave = wave;
  x.lane = lane;
  x.nchunks = (x.g1 - x.g0 + CGW - 1) / CGW;
  // the A rows this wave stages: rows that do not exist are not loaded (their
  // LDS rows hold stale data, which only reaches output rows never stored)
  const int rows_used = MOE ? 16 : (p.M < 16 ? p.M : 16);
  x.stage_a = 2 * wave < rows_used;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int row = 2 * wave + h;
    row = row < rows_used ? row : rows_used - 1;
    int src = row;
    if constexpr (MOE) {
      const int id = p.sorted_ids[mb * 16 + row];
      src = id < p.num_pairs ? (p.a_per_pair ? id : id / p.top_k) : 0;
    }
    x.arow[h] = (const char*)p.A + (size_t)src * p.K * 2 + lane * 16;
  }

  uint32_t um;
  asm volatile("v_mov_b32 %0, %1" : "=v"(um) : "s"(p.unpack_mask));
  const uint32_t ue = p.unpack_exp;

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  WsChunkRegs rA, rB;
  ws_issue(rA, x, x.g0);  // prologue: chunk 0 in flight
  // chunks in pairs (buffer 0, buffer 1); the last chunk starts nothing
  int i = 0;
  for (; i + 2 < x.nchunks; i += 2) {
    ws_chunk<ASYM, 0, true>(x, i, rA, rB, acc, um, ue);
    ws_chunk<ASYM, 1, true>(x, i + 1, rB, rA, acc, um, ue);
  }
  if (i + 1 < x.nchunks) {
    ws_chunk<ASYM, 0, true>(x, i, rA, rB, acc, um, ue);
    ws_chunk<ASYM, 1, false>(x, i + 1, rB, rA, acc, um, ue);
  } else {
    ws_chunk<ASYM, 0, false>(x, i, rA, rB, acc, um, ue);
  }

  // add the two K halves in a fixed order: half 1 parks its sums in LDS
  __syncthreads();
  float* park = (float*)ws_lds0;  // [NT][16 rows][16 cols]
  if (kp == 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) park[(t * 16 + 4 * c + e) * 16 + col] = acc[e];
  }
  __syncthreads();
  if (kp == 1 || tile >= p.ntiles) return;
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] += park[(t * 16 + 4 * c + e) * 16 + col];

  ws_store<MOE>(p, acc, tile, split, mb, c, col);
}

// ---------------------------------------------------------------------------
// Resident-A variant: when a workgroup's K range holds at most 32 groups, its
// A rows (16 x 32 x 128 bf16 = 128 KiB), its scale records and the row sums
// of every group are put into LDS once, up front; after that each wave only
// streams its weight units through a ring of RU registers, with no further
// synchronisation until the K halves are added. The prologue loads go through
// registers too (no direct-to-LDS copies), so the compiler's waits let the
// first weight units stay in flight while the A rows are staged.
constexpr int RG = 32;                     // groups per workgroup at most
constexpr int RGW = RG / KW;               // per wave (16)
constexpr int RU = 8;                      // weight units in flight per wave
constexpr int R_PITCH = RG * 256 + 16;     // 8208-byte LDS rows
constexpr int R_A = 16 * R_PITCH;
constexpr int RAL = RG * 256 / 1024;       // 16-byte loads per lane per A row (8)
constexpr int R_S = WAVES * RGW * 128;
constexpr int R_C = RG * 16 * 4;
constexpr int R_LDS = R_A + R_S + R_C;
static_assert(R_LDS <= 160 * 1024, "fits the LDS of one CU");
static_assert(RGW * 128 == 2 * 1024, "two record loads per wave");

__shared__ __attribute__((aligned(1024))) char wsr_lds[R_LDS];

template <bool ASYM, bool MOE>
__global__ __launch_bounds__(512) void wsr_kernel(const GemmArgs p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane >> 4, col = lane & 15;
  const int t = wave % NT, kp = wave / NT;
  const int nb = blockIdx.x, split = blockIdx.y, mb = blockIdx.z;

  int expert = 0;
  if constexpr (MOE) {
    if (mb * 16 >= *p.num_padded) return;
    expert = p.block_expert[mb];
  }
  const uint8_t* wbase = p.packed + (size_t)expert * p.expert_stride;
  const int groups = p.groups;
  const int tile = nb * NT + t;
  const int ltile = tile < p.ntiles ? tile : p.ntiles - 1;  // clamped (never stored)
  const int g0 = (int)(((int64_t)split * groups) / gridDim.y);
  const int g1 = (int)(((int64_t)(split + 1) * groups) / gridDim.y);
  const int gsz = g1 - g0;                 // <= RG (checked by the host)
  const int half = (gsz + 1) / 2;
  const int hg0 = g0 + kp * half;          // this wave's groups [hg0, hg0 + cnt)
  const int cnt = min(half, g1 - hg0);

  // ---- prologue loads: A rows 2w, 2w+1 (those that exist; the other LDS
  // rows keep stale data, which only reaches output rows never stored), this
  // wave's scale records, its first RU weight units
  const int rows_used = MOE ? 16 : (p.M < 16 ? p.M : 16);
  const bool stage_a = 2 * wave < rows_used;
  u32x4_t ar[2][RAL];
  if (stage_a) {  // wave-uniform
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int row = 2 * wave + h;
      row = row < rows_used ? row : rows_used - 1;
      int src = row;
      if constexpr (MOE) {
        const int id = p.sorted_ids[mb * 16 + row];
        src = id < p.num_pairs ? (p.a_per_pair ? id : id / p.top_k) : 0;
      }
      const char* arow = (const char*)p.A + (size_t)src * p.K * 2 + (size_t)g0 * 256;
#pragma unroll
      for (int k = 0; k < RAL; ++k) {
        const int slot = k * 64 + lane;  // 16-byte slot of the range; past it: slot 0
        ar[h][k] = *(const u32x4_t*)(arow + (slot < gsz * 16 ? slot : 0) * 16);
      }
    }
  }
  const uint8_t* srec = wbase + p.s_offset + (size_t)ltile * groups * 128;
  u32x4_t sr[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    int g = hg0 + (k * 64 + lane) / 8;
    g = g < g1 ? g : g1 - 1;
    sr[k] = *(const u32x4_t*)(srec + (size_t)g * 128 + (lane & 7) * 16);
  }
  const uint8_t* wt = wbase + (size_t)ltile * groups * kUnit4Bytes + lane * 16;
  u32x4_t ring[RU];
#pragma unroll
  for (int u = 0; u < RU; ++u) {
    const int g = hg0 + (u < cnt ? u : cnt - 1);
    ring[u] = ldg_nt((const u32x4_t*)(wt + (size_t)g * kUnit4Bytes));
  }
  if (stage_a) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int k = 0; k < RAL; ++k) *(u32x4_t*)(wsr_lds + (2 * wave + h) * R_PITCH + (k * 64 + lane) * 16) = ar[h][k];
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) *(u32x4_t*)(wsr_lds + R_A + wave * (RGW * 128) + k * 1024 + lane * 16) = sr[k];
  ws_barrier();

  // row sums of every group of the range (pre-scaled by -136 when symmetric)
  float* corr = (float*)(wsr_lds + R_A + R_S);
#pragma unroll
  for (int h = 0; h < RG / WAVES; ++h) {
    const int q = wave + h * WAVES;
    f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    const u32x4_t kb = ASYM ? u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u}   // bf16 1.0
                            : u32x4_t{0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u};  // bf16 -136
#pragma unroll
    for (int j = 0; j < 4; ++j)
      z = mfma_bf16(*(const u32x4_t*)(wsr_lds + col * R_PITCH + q * 256 + (4 * c + j) * 16), kb, z);
    if (col == 0) *(f32x4_t*)(corr + q * 16 + 4 * c) = z;
  }
  ws_barrier();

  uint32_t um;
  asm volatile("v_mov_b32 %0, %1" : "=v"(um) : "s"(p.unpack_mask));
  const uint32_t ue = p.unpack_exp;
  const char* srecs = wsr_lds + R_A + wave * (RGW * 128);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  // the ring: unit u is computed, then unit u + RU takes its registers; every
  // unit is computed (straight-line code keeps the load waits exact) and
  // units past cnt (in-bounds re-reads, finite) are dropped by a select
#pragma unroll
  for (int u = 0; u < RGW; ++u) {
    const int q = hg0 - g0 + u;  // group within the range
    u32x4_t a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = *(const u32x4_t*)(wsr_lds + col * R_PITCH + q * 256 + (4 * c + j) * 16);
    const f32x4_t rs = *(const f32x4_t*)(corr + q * 16 + 4 * c);
    const u32x2_t rec = *(const u32x2_t*)(srecs + u * 128 + col * 8);
    f32x4_t pacc;
    if constexpr (ASYM) {
      const float negz = __builtin_bit_cast(float, (rec.y & 0xFFFFu) << 16);  // -(128+z)
      pacc = f32x4_t{negz * rs[0], negz * rs[1], negz * rs[2], negz * rs[3]};
    } else {
      pacc = rs;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) pacc = mfma_bf16(a[j], unpack_u4_bf16_offset128(ring[u % RU][j], um, ue), pacc);
    const float s = bits_as<float>(rec.x);
    if (u + RU < RGW) {
      const int g = hg0 + (u + RU < cnt ? u + RU : cnt - 1);
      ring[u % RU] = ldg_nt((const u32x4_t*)(wt + (size_t)g * kUnit4Bytes));
    }
    const bool valid = u < cnt;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = valid ? __builtin_fmaf(s, pacc[e], acc[e]) : acc[e];
  }

  // add the two K halves in a fixed order: half 1 parks its sums in LDS
  __syncthreads();
  float* park = (float*)wsr_lds;  // [NT][16 rows][16 cols]
  if (kp == 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) park[(t * 16 + 4 * c + e) * 16 + col] = acc[e];
  }
  __syncthreads();
  if (kp == 1 || tile >= p.ntiles) return;
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] += park[(t * 16 + 4 * c + e) * 16 + col];
  ws_store<MOE>(p, acc, tile, split, mb, c, col);
}

#ifndef __HIPCC_RTC__  // host launchers
template <bool ASYM, bool MOE>
hipError_t launch_ws(const GemmArgs& a, int nsplit, int grid_m, hipStream_t s, KernelLaunch* d) {
  dim3 grid((a.ntiles + NT - 1) / NT, nsplit, grid_m);
  const bool resident = (a.groups + nsplit - 1) / nsplit <= RG;
  if (d) {
    d->src = JIT_SRC_WSTREAM;
    std::snprintf(d->expr, sizeof d->expr, "qdg::%s<%s, %s>", resident ? "wsr_kernel" : "wstream_kernel",
                  ASYM ? "true" : "false", MOE ? "true" : "false");
    d->grid[0] = grid.x;
    d->grid[1] = grid.y;
    d->grid[2] = grid.z;
    d->block = 64 * WAVES;
    d->mn_args = false;
    return hipSuccess;
  }
  if (resident)
    hipLaunchKernelGGL((wsr_kernel<ASYM, MOE>), grid, dim3(64 * WAVES), 0, s, a);
  else
    hipLaunchKernelGGL((wstream_kernel<ASYM, MOE>), grid, dim3(64 * WAVES), 0, s, a);
  return hipGetLastError();
}

#endif  // __HIPCC_RTC__
}  // namespace

#ifndef __HIPCC_RTC__  // host launchers
hipError_t launch_wstream(bool asym, bool moe, const GemmArgs& a, int nsplit, int grid_m, hipStream_t s,
                          KernelLaunch* d) {
  if (moe) return asym ? hipErrorInvalidValue : launch_ws<false, true>(a, 1, grid_m, s, d);
  hipError_t e = asym ? launch_ws<true, false>(a, nsplit, 1, s, d) : launch_ws<false, false>(a, nsplit, 1, s, d);
  if (!d && e == hipSuccess && nsplit > 1) e = launch_reduce_splits(a, 16, a.ntiles * 16, s);
  return e;
}

#endif  // __HIPCC_RTC__

}  // namespace qdg
