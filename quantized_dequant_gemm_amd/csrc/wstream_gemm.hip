// Weight-streaming W4A16 kernel for M <= 16 (dense) and for the grouped MoE
// GEMM when an expert block holds at most 16 rows.
//
// At this size the layer is a stream of packed weights from HBM; everything
// else is arranged so that the stream starts at once and never waits:
//   * a 256-thread workgroup (one per CU) owns four 16-column N tiles, one per
//     wavefront, over a K range that it walks in chunks of up to 32 groups;
//   * per chunk, each wave issues all its weight loads at once (32 coalesced
//     1 KiB units = 128 VGPRs in flight per wave), right after the chunk's A
//     rows (16 x 32 x 128 bf16) and scale records were requested by direct
//     global -> LDS copies; the A rows are shared by the four waves from LDS;
//   * the MFMA chains of a group start from -(128+z) * rowsum(A), computed
//     once per group by one wave (the streaming family's offset trick);
//   * when the N tiles alone cannot occupy the CUs (4096-wide down
//     projections) K is split across workgroups and reduce_splits_kernel adds
//     the fp32 partials in split order (deterministic, no device fences).
// The pages' small-batch pipeline streams weights through a multi-stage
// asynchronous copy (kinachrichten, "Wie die Architektur funktioniert");
// direct LDS copies plus a full chunk of register-resident loads is the gfx950
// form of that idea.
#include "qdg_device.h"
#include "qdg_internal.h"

namespace qdg {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int GS = 32;                      // groups per chunk (max)
constexpr int A_PITCH = GS * 256 + 16;      // padded LDS row: conflict-free fragment reads
constexpr int A_SLOTS_ROW = A_PITCH / 16;   // 513
constexpr int A_INST = (16 * A_SLOTS_ROW + 63) / 64;  // 129 wave copies per chunk
// the last copy's lanes past row 15 land in the tail of this area (unread)
constexpr int A_BYTES = A_INST * 1024;
static_assert(A_BYTES >= 16 * A_PITCH, "A area holds the 16 padded rows");
constexpr int SC_BYTES = GS * 128;          // scale records of one tile for one chunk
constexpr int CORR_BYTES = GS * 16 * 4;
constexpr int SMEM = A_BYTES + 4 * SC_BYTES + CORR_BYTES;

// DMA of one chunk: A rows and the wave's scale records. The copy plan is
// fixed for the whole kernel: wave copy i moves slot q = 64 i + lane of the
// padded A tile, i.e. row q / 513, 16-byte chunk q % 513 (chunks past the
// chunk's groups re-read chunk 0); plan[r] packs the source row index (low
// 21 bits) and the chunk (high bits). Out of lambdas on purpose (device-only
// builtins).
constexpr int DMA_PER_WAVE = (A_INST + 3) / 4;

__device__ __forceinline__ void wstream_dma(char* smem, const char* a, size_t a_row_bytes, const uint32_t* plan,
                                            int wave, int lane, int cg0, int gs, const uint8_t* srec, int sc_off) {
  const char* ag = a + (size_t)cg0 * 256;
#pragma unroll
  for (int r = 0; r < DMA_PER_WAVE; ++r) {
    const int i = r * 4 + wave;
    if (i < A_INST) {
      const uint32_t src = plan[r] & 0x1FFFFFu, ch = plan[r] >> 21;
      const uint32_t gch = ch < (uint32_t)gs * 16 ? ch : 0;
      __builtin_amdgcn_global_load_lds(ag + (size_t)src * a_row_bytes + gch * 16, (lds_void*)(smem + i * 1024), 16,
                                       0, 0);
    }
  }
#pragma unroll
  for (int k = 0; k < SC_BYTES / 1024; ++k) {
    if (k * 1024 + lane * 16 < gs * 128)
      __builtin_amdgcn_global_load_lds(srec + k * 1024 + lane * 16, (lds_void*)(smem + sc_off + k * 1024), 16, 0,
                                       0);
  }
}

template <bool ASYM, bool MOE>
__global__ __launch_bounds__(256) void wstream_kernel(const GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane >> 4, col = lane & 15;
  const int nb = blockIdx.x, split = blockIdx.y, mb = blockIdx.z;

  int expert = 0;
  if constexpr (MOE) {
    if (mb * 16 >= *p.num_padded) return;
    expert = p.block_expert[mb];
  }
  const uint8_t* wbase = p.packed + (size_t)expert * p.expert_stride;
  const uint8_t* sbase = wbase + p.s_offset;
  const int groups = p.groups;
  const int tile = nb * 4 + wave;
  const int ltile = tile < p.ntiles ? tile : p.ntiles - 1;  // clamped (never stored)

  // copy plan of this lane (see wstream_dma)
  uint32_t plan[DMA_PER_WAVE];
#pragma unroll
  for (int r = 0; r < DMA_PER_WAVE; ++r) {
    const int q = (r * 4 + wave) * 64 + lane;
    int row = q / A_SLOTS_ROW;
    const int ch = q - row * A_SLOTS_ROW;
    row = row < 16 ? row : 15;
    int src;
    if constexpr (MOE) {
      const int id = p.sorted_ids[mb * 16 + row];
      src = id < p.num_pairs ? (p.a_per_pair ? id : id / p.top_k) : 0;
    } else {
      src = row < p.M ? row : p.M - 1;
    }
    plan[r] = (uint32_t)src | ((uint32_t)ch << 21);
  }
  const size_t a_row_bytes = (size_t)p.K * 2;

  const int g0 = (int)(((int64_t)split * groups) / gridDim.y);
  const int g1 = (int)(((int64_t)(split + 1) * groups) / gridDim.y);
  const int sc_off = A_BYTES + wave * SC_BYTES;
  float* corr = (float*)(smem + A_BYTES + 4 * SC_BYTES);
  uint32_t um;
  asm volatile("v_mov_b32 %0, %1" : "=v"(um) : "s"(p.unpack_mask));
  const uint32_t ue = p.unpack_exp;

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int cg0 = g0; cg0 < g1; cg0 += GS) {
    const int gs = min(GS, g1 - cg0);
    __syncthreads();  // the previous chunk's LDS is no longer read
    wstream_dma(smem, (const char*)p.A, a_row_bytes, plan, wave, lane, cg0, gs,
                sbase + ((size_t)ltile * groups + cg0) * 128, sc_off);
    asm volatile("" ::: "memory");  // copies first, then the weight loads (vmcnt order)
    // all GS weight loads, always issued (units past the chunk re-read unit 0)
    u32x4_t b[GS];
    const u32x4_t* wt = (const u32x4_t*)(wbase + ((size_t)ltile * groups + cg0) * kUnit4Bytes) + lane;
#pragma unroll
    for (int u = 0; u < GS; ++u) b[u] = ldg_nt(wt + (u < gs ? u : 0) * 64);
    asm volatile("" ::: "memory");
    // this wave's copies have landed once at most the GS weight loads remain
    __builtin_amdgcn_s_waitcnt((GS & 15) | (7 << 4) | (15 << 8) | ((GS >> 4) << 14));
    __syncthreads();
    // per-group row sums of A (pre-scaled by -136 when symmetric), one wave per group
    for (int u = wave; u < gs; u += 4) {
      f32x4_t z = {0.f, 0.f, 0.f, 0.f};
      const u32x4_t kb = ASYM ? u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u}   // bf16 1.0
                              : u32x4_t{0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u};  // bf16 -136
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4_t a = *(const u32x4_t*)(smem + col * A_PITCH + u * 256 + (4 * c + j) * 16);
        z = mfma_bf16(a, kb, z);
      }
      if (col == 0) *(f32x4_t*)(corr + u * 16 + 4 * c) = z;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < GS; ++u) {
      if (u < gs) {  // wave-uniform
        u32x4_t a[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] = *(const u32x4_t*)(smem + col * A_PITCH + u * 256 + (4 * c + j) * 16);
        const f32x4_t rs = *(const f32x4_t*)(corr + u * 16 + 4 * c);
        const u32x2_t rec = *(const u32x2_t*)(smem + sc_off + u * 128 + col * 8);
        f32x4_t pacc;
        if constexpr (ASYM) {
          const float negz = __builtin_bit_cast(float, (rec.y & 0xFFFFu) << 16);  // -(128+z)
          pacc = f32x4_t{negz * rs[0], negz * rs[1], negz * rs[2], negz * rs[3]};
        } else {
          pacc = rs;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) pacc = mfma_bf16(a[j], unpack_u4_bf16_offset128(b[u][j], um, ue), pacc);
        const float s = bits_as<float>(rec.x);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(s, pacc[i], acc[i]);
      }
    }
  }

  // ---- output: lane holds rows 4c+i of column `col` of its tile
  if (tile >= p.ntiles) return;
  const int n = tile * 16 + col;
  if (gridDim.y > 1) {  // fp32 partial [split][16][n_pad]
    const int n_pad = p.ntiles * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) ((float*)p.partial)[((size_t)split * 16 + 4 * c + i) * n_pad + n] = acc[i];
    return;
  }
  if (n >= p.N) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * c + i;
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
      ((float*)p.Y)[o] = acc[i];
    else
      ((uint16_t*)p.Y)[o] = (uint16_t)f32_to_bf16_rne(acc[i]);
  }
}

template <bool ASYM, bool MOE>
hipError_t launch_ws(const GemmArgs& a, int nsplit, int grid_m, hipStream_t s) {
  static bool attr_set = false;  // idempotent; a race only repeats the call
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&wstream_kernel<ASYM, MOE>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, SMEM);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid((a.ntiles + 3) / 4, nsplit, grid_m);
  hipLaunchKernelGGL((wstream_kernel<ASYM, MOE>), grid, dim3(256), SMEM, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_wstream(bool asym, bool moe, const GemmArgs& a, int nsplit, int grid_m, hipStream_t s) {
  if (moe) return asym ? hipErrorInvalidValue : launch_ws<false, true>(a, 1, grid_m, s);
  hipError_t e = asym ? launch_ws<true, false>(a, nsplit, 1, s) : launch_ws<false, false>(a, nsplit, 1, s);
  if (e == hipSuccess && nsplit > 1) e = launch_reduce_splits(a, 16, a.ntiles * 16, s);
  return e;
}

}  // namespace qdg
