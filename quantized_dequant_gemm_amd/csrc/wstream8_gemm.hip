// Weight-streaming kernel for the 8-bit-activation formats at M <= 16:
// W8A8 and W4A8-INT8 (v_mfma_i32_16x16x64_i8) and W4A8-MXFP4 (scaled
// fp8 x fp4 MFMA, E8M0 block scales applied by the hardware).
//
// The same design as the W4A16 resident-A weight-streaming kernel: at this
// size the layer is a stream of packed weights from HBM (the pages' small-
// batch pipeline, kinachrichten "Wie die Architektur funktioniert"), so
//   * a workgroup of 8 waves owns 4 adjacent 16-column N tiles and a K range
//     of at most 64 groups; wave w works on tile w % 4 and half w / 4 of it;
//   * the A rows of the range (16 x 64 x 128 bytes), the wave's per-group
//     weight records and (fp8) the activation scales are put into LDS once,
//     then each wave streams its weight units through a ring of 8 loads in
//     flight with no further synchronisation;
//   * W8A8 accumulates exact int32 and applies token and channel scales in
//     the epilogue; W4A8 adds s * P per group in fp32 (int32 in raw mode);
//     MXFP4 adds a_scale * P per group;
//   * the two K halves are added through LDS in a fixed order; K splits
//     across workgroups only to occupy the CUs, reduced by
//     reduce_splits_kernel in split order.
#ifndef __HIPCC_RTC__
#include <cstdio>
#include <type_traits>
#endif

#include "qdg_device.h"
#include "qdg_internal.h"

namespace qdg {
namespace {

enum W8Kind { K_W8A8 = 0, K_W4A8 = 1, K_MXFP4 = 2 };

// A workgroup has 8 waves: NT N tiles x KW = 8 / NT parts of its K range
// (NT = 4 for wide layers; NT = 1 when there are too few tiles to occupy the
// CUs, which avoids splitting K across workgroups).
constexpr int WAVES = 8;
constexpr int RG = 64;                   // groups per workgroup at most
constexpr int PITCH = RG * 128 + 16;     // 8208-byte LDS rows of A
constexpr int L_A = 16 * PITCH;
constexpr int RAL = RG * 128 / 1024;     // 16-byte loads per lane per A row (8)
constexpr int REC_W = 2048;              // per wave: up to 32 groups x 64 bytes of records
constexpr int L_REC = L_A;
constexpr int L_AS = L_REC + WAVES * REC_W;  // fp8: [group][16 rows] activation scales
constexpr int L_BYTES = L_AS + RG * 16 * 4;
static_assert(L_BYTES <= 160 * 1024, "fits the LDS of one CU");
static_assert(7 * 256 * 4 <= L_A, "the K-part exchange fits the A area");

__shared__ __attribute__((aligned(1024))) char w8_lds[L_BYTES];

__device__ __forceinline__ void w8_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); loads in flight stay in flight
  asm volatile("s_barrier" ::: "memory");
}

template <int KIND, bool RAW>
struct W8Acc {
  using T = typename std::conditional<KIND == K_W8A8 || RAW, i32x4_t, f32x4_t>::type;
};

template <int KIND, bool RAW, int NT>
__global__ __launch_bounds__(512) void wsr8_kernel(const GemmArgs p) {
  constexpr int KW = WAVES / NT;              // K parts
  constexpr int RGW = RG / KW;                // groups per wave at most
  constexpr int SRL = (RGW * 64 + 1023) / 1024;  // record loads per lane
  static_assert(RGW * 64 <= REC_W, "records of a wave fit its LDS slice");
  constexpr int UL = KIND == K_W8A8 ? 2 : 1;  // 16-byte loads per lane per weight unit
  constexpr int UB = UL * 1024;               // bytes per unit
  constexpr int RU = 8 / UL;                  // units in flight per wave (8 loads)
  using Acc = typename W8Acc<KIND, RAW>::T;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane >> 4, col = lane & 15;
  const int t = wave % NT, kp = wave / NT;
  const int nb = blockIdx.x, split = blockIdx.y;

  const uint8_t* wbase = p.packed;
  const uint8_t* sbase = wbase + p.s_offset;
  const int groups = p.groups;
  const int tile = nb * NT + t;
  const int ltile = tile < p.ntiles ? tile : p.ntiles - 1;  // clamped (never stored)
  const int g0 = (int)(((int64_t)split * groups) / gridDim.y);
  const int g1 = (int)(((int64_t)(split + 1) * groups) / gridDim.y);
  const int gsz = g1 - g0;  // <= RG (checked by the host)
  const int per = (gsz + KW - 1) / KW;
  const int hg0 = g0 + kp * per;  // this wave's groups [hg0, hg0 + cnt); cnt may be <= 0
  const int cnt = min(per, g1 - hg0);
  // unit u of this wave reads group wg(u) (past cnt: a valid group, unused)
  auto wg = [&](int u) { return max(min(hg0 + min(u, cnt - 1), g1 - 1), g0); };
  const int rows_used = p.M < 16 ? p.M : 16;

  // ---- prologue: A rows 2w, 2w+1 (rows that do not exist are not loaded:
  // their LDS rows keep stale data, which only reaches rows never stored),
  // the wave's records, the first RU units; fp8: the activation scales
  const bool stage_a = 2 * wave < rows_used;
  u32x4_t ar[2][RAL];
  if (stage_a) {  // wave-uniform
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = min(2 * wave + h, rows_used - 1);
      const char* arow = (const char*)p.A + (size_t)row * p.K + (size_t)g0 * 128;
#pragma unroll
      for (int k = 0; k < RAL; ++k) {
        const int slot = k * 64 + lane;  // 16-byte slot of the range; past it: slot 0
        ar[h][k] = *(const u32x4_t*)(arow + (slot < gsz * 8 ? slot : 0) * 16);
      }
    }
  }
  u32x4_t sr[SRL];
  if constexpr (KIND != K_W8A8) {
    // records of unit (tile, group): 64 bytes (W4A8: 16 x f32 s/16; MXFP4: E8M0 per lane)
    const uint8_t* srec = sbase + (size_t)ltile * groups * 64;
#pragma unroll
    for (int k = 0; k < SRL; ++k) {
      const int g = wg((k * 64 + lane) / 4);
      sr[k] = *(const u32x4_t*)(srec + (size_t)g * 64 + (lane & 3) * 16);
    }
  }
  float asv[2];
  if constexpr (KIND == K_MXFP4) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = h * 512 + threadIdx.x;  // [group q][row]
      const int q = e / 16, row = min(e % 16, rows_used - 1);
      asv[h] = q < gsz ? p.a_scales[(size_t)row * groups + g0 + q] : 0.f;
    }
  }
  const uint8_t* wt = wbase + (size_t)ltile * groups * UB + lane * 16;
  u32x4_t ring[RU][UL];
#pragma unroll
  for (int u = 0; u < RU; ++u) {
    const int g = wg(u);
#pragma unroll
    for (int h = 0; h < UL; ++h) ring[u][h] = ldg_nt((const u32x4_t*)(wt + (size_t)g * UB + h * 1024));
  }
  if (stage_a) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int k = 0; k < RAL; ++k) *(u32x4_t*)(w8_lds + (2 * wave + h) * PITCH + (k * 64 + lane) * 16) = ar[h][k];
  }
  if constexpr (KIND != K_W8A8) {
#pragma unroll
    for (int k = 0; k < SRL; ++k)
      if (k * 1024 + lane * 16 < REC_W) *(u32x4_t*)(w8_lds + L_REC + wave * REC_W + k * 1024 + lane * 16) = sr[k];
  }
  if constexpr (KIND == K_MXFP4) {
#pragma unroll
    for (int h = 0; h < 2; ++h) ((float*)(w8_lds + L_AS))[h * 512 + threadIdx.x] = asv[h];
  }
  w8_barrier();

  // ---- the ring: unit u is computed, then unit u + RU takes its registers;
  // every unit is computed (straight-line code keeps the load waits exact)
  // and units past cnt (in-bounds re-reads, finite) are dropped by a select
  const char* recs = w8_lds + L_REC + wave * REC_W;
  Acc acc = {0, 0, 0, 0};
#pragma unroll
  for (int u = 0; u < RGW; ++u) {
    const int q = hg0 - g0 + u;  // group within the range
    const bool valid = u < cnt;
    const char* ap = w8_lds + col * PITCH + q * 128;
    const u32x4_t a0 = *(const u32x4_t*)(ap + (KIND == K_MXFP4 ? 16 : 32) * c);
    const u32x4_t a1 = *(const u32x4_t*)(ap + (KIND == K_MXFP4 ? 16 * c + 64 : 32 * c + 16));
    if constexpr (KIND == K_W8A8) {
      const i32x4_t r = mfma_i8(a1, ring[u % RU][1], mfma_i8(a0, ring[u % RU][0], acc));
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = valid ? r[e] : acc[e];
    } else if constexpr (KIND == K_W4A8) {
      const u32x4_t x = ring[u % RU][0];
      const u32x2_t l0 = unpack_i4_i8x16(x.x), h0 = unpack_i4_i8x16(x.y);
      const u32x2_t l1 = unpack_i4_i8x16(x.z), h1 = unpack_i4_i8x16(x.w);
      const i32x4_t pr = mfma_i8(a1, u32x4_t{l1.x, l1.y, h1.x, h1.y},
                                 mfma_i8(a0, u32x4_t{l0.x, l0.y, h0.x, h0.y}, i32x4_t{0, 0, 0, 0}));
      if constexpr (RAW) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += valid ? pr[e] : 0;
      } else {
        const float ws = valid ? *(const float*)(recs + u * 64 + col * 4) : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(ws, (float)pr[e], acc[e]);
      }
    } else {
      const int e8 = *(const uint8_t*)(recs + u * 64 + lane);
      const f32x4_t as = *(const f32x4_t*)(w8_lds + L_AS + (q * 16 + 4 * c) * 4);
      const u32x4_t b = ring[u % RU][0];
      const i32x8_t av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      const i32x8_t bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
      const f32x4_t pr = mfma_fp8_fp4_scaled(av, bv, f32x4_t{0.f, 0.f, 0.f, 0.f}, 127, e8);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = valid ? __builtin_fmaf(as[e], pr[e], acc[e]) : acc[e];
    }
    if (u + RU < RGW) {
      const int g = wg(u + RU);
#pragma unroll
      for (int h = 0; h < UL; ++h) ring[u % RU][h] = ldg_nt((const u32x4_t*)(wt + (size_t)g * UB + h * 1024));
    }
  }

  // ---- add the K parts in a fixed order: parts 1..KW-1 park their sums in
  // LDS, part 0 adds them in order
  __syncthreads();
  uint32_t* park = (uint32_t*)w8_lds;  // [KW-1][NT][16 rows][16 cols]
  if (kp > 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      park[(((kp - 1) * NT + t) * 16 + 4 * c + e) * 16 + col] = bits_as<uint32_t>(acc[e]);
  }
  __syncthreads();
  if (kp > 0 || tile >= p.ntiles) return;
#pragma unroll
  for (int j = 1; j < KW; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t v = park[(((j - 1) * NT + t) * 16 + 4 * c + e) * 16 + col];
      if constexpr (KIND == K_W8A8 || RAW)
        acc[e] += (int)v;
      else
        acc[e] += __builtin_bit_cast(float, v);
    }

  // ---- epilogue: lane holds rows 4c+e of column `col` of its tile
  const int n = tile * 16 + col;
  const bool raw = p.otype == QDG_O_I32;
  float sw = 1.f;
  if constexpr (KIND == K_W8A8) sw = ((const float*)sbase)[tile * 16 + col];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = 4 * c + e;
    if (r >= p.M) continue;
    float y;
    // raw int32 output takes no scale: a_scales may be NULL then
    if constexpr (KIND == K_W8A8)
      y = RAW ? 0.f : (float)acc[e] * p.a_scales[r] * sw;
    else if constexpr (KIND == K_W4A8)
      y = RAW ? 0.f : (float)acc[e] * p.a_scales[r];
    else
      y = acc[e];
    if (gridDim.y > 1) {  // fp32 partial [split][16][n_pad] (never raw)
      ((float*)p.partial)[((size_t)split * 16 + r) * (p.ntiles * 16) + n] = y;
      continue;
    }
    if (n >= p.N) continue;
    const size_t o = (size_t)r * p.N + n;
    if (raw) {
      int v = bits_as<int>(acc[e]);
      if constexpr (KIND == K_W4A8) v >>= 4;  // 16 q * qa: exact shift back
      ((int*)p.Y)[o] = v;
    } else if (p.otype == QDG_O_F32) {
      ((float*)p.Y)[o] = y;
    } else {
      ((uint16_t*)p.Y)[o] = (uint16_t)f32_to_bf16_rne(y);
    }
  }
}

#ifndef __HIPCC_RTC__  // host launchers
template <int KIND, bool RAW>
hipError_t launch_w8(const GemmArgs& a, int nsplit, int nt, hipStream_t s, KernelLaunch* d) {
  if (d) {
    d->src = JIT_SRC_WSTREAM8;
    std::snprintf(d->expr, sizeof d->expr, "qdg::wsr8_kernel<%d, %s, %d>", KIND, RAW ? "true" : "false", nt);
    d->grid[0] = (unsigned)(nt == 1 ? a.ntiles : (a.ntiles + 3) / 4);
    d->grid[1] = (unsigned)nsplit;
    d->grid[2] = 1;
    d->block = 64 * WAVES;
    d->mn_args = false;
    return hipSuccess;
  }
  if (nt == 1) {
    hipLaunchKernelGGL((wsr8_kernel<KIND, RAW, 1>), dim3(a.ntiles, nsplit, 1), dim3(64 * WAVES), 0, s, a);
  } else {
    hipLaunchKernelGGL((wsr8_kernel<KIND, RAW, 4>), dim3((a.ntiles + 3) / 4, nsplit, 1), dim3(64 * WAVES), 0, s, a);
  }
  return hipGetLastError();
}

#endif  // __HIPCC_RTC__
}  // namespace

#ifndef __HIPCC_RTC__  // host launchers
// Largest K range (in 128-wide groups) one workgroup of this family holds.
int wstream8_max_groups() { return RG; }

hipError_t launch_wstream8(Format f, const GemmArgs& a, int nsplit, int nt, hipStream_t s, KernelLaunch* d) {
  const bool raw = a.otype == QDG_O_I32;
  if ((a.groups + nsplit - 1) / nsplit > RG || (raw && nsplit > 1) || (nt != 1 && nt != 4))
    return hipErrorInvalidValue;
  hipError_t e;
  switch (f) {
    case FMT_W8A8: e = raw ? launch_w8<K_W8A8, true>(a, 1, nt, s, d) : launch_w8<K_W8A8, false>(a, nsplit, nt, s, d); break;
    case FMT_W4A8: e = raw ? launch_w8<K_W4A8, true>(a, 1, nt, s, d) : launch_w8<K_W4A8, false>(a, nsplit, nt, s, d); break;
    case FMT_MXFP4: e = launch_w8<K_MXFP4, false>(a, nsplit, nt, s, d); break;
    default: return hipErrorInvalidValue;
  }
  if (!d && e == hipSuccess && nsplit > 1) e = launch_reduce_splits(a, 16, a.ntiles * 16, s);
  return e;
}

#endif  // __HIPCC_RTC__

}  // namespace qdg
