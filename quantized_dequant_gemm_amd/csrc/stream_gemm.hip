// Streaming (small-M) GEMM family for gfx950.
//
// The pages' library runs small batches on a deep multi-stage pipeline that
// streams weights, and large batches on a different, tile-oriented pipeline
// (kinachrichten, "Wie die Architektur funktioniert"). At small M the layer is
// bound by the HBM stream of packed weights, so this family is organised
// around that stream:
//   * a workgroup owns NT 16-column N tiles, MT 16-row M tiles and one of
//     `split` K partitions; its KW wavefronts interleave over the K groups of
//     the partition (wave w takes groups g0+w, g0+w+KW, ...), so at any time
//     the workgroup reads KW adjacent 1 KiB units of each tile;
//   * each unit is one fully coalesced 16-byte-per-lane load; loads for the
//     next U groups are issued before the current ones are consumed (register
//     double buffering) to keep enough bytes in flight per CU;
//   * dequantization happens in registers right before the MFMA;
//   * the KW wave partials are reduced through LDS in a fixed order; with
//     `split` > 1 every workgroup writes its fp32 partial into the caller's
//     workspace and reduce_splits_kernel adds the partitions in split order,
//     so results are deterministic.
// The five component roles the pages name for their CUDA layer (scheduling,
// data movement, dequantization and scaling, matrix-core compute, output
// processing; kinachrichten, "Kompilierzeiten und gerätespezifisches Tuning")
// map to: the grid/wave-to-unit mapping, Fmt::load, Fmt::compute, the MFMA
// wrappers, and epilogue().
#ifndef __HIPCC_RTC__
#include <type_traits>
#endif

#include "qdg_device.h"
#include "qdg_internal.h"

namespace qdg {
namespace {

// ----------------------------------------------------------------- policies
// Every policy defines Frag<MT,NT> (the registers of one K group), Acc (the
// accumulator type), load(), compute() and value() (final scaling of one
// accumulator element into the output domain).

constexpr uint32_t kAOob = 0x80000000u;  // past every A (the host keeps A < 2^31 bytes)

__device__ __forceinline__ u32x4_t lda(const __amdgpu_buffer_rsrc_t& r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

struct Ctx {
  // A through a buffer resource: the byte offset of this lane's row for each
  // M tile, or kAOob for a padding row, whose loads then return zeros without
  // a memory access (the load is still issued, so every path issues the same
  // loads)
  __amdgpu_buffer_rsrc_t arsrc;
  uint32_t aoff[4];
  int as_row[4][4];      // A row of the D rows 4c+i of each M tile (fp8 activation scales)
  int arow_s[4];         // A row of this lane for each M tile, 0 for padding rows (fp4 activation scales)
  const uint8_t* a_e8m0; // fp4 activation scales (E8M0 per row and 32-block)
  const uint8_t* wbase;  // weight units of this expert
  const uint8_t* sbase;  // scale records of this expert
  const float* a_scales; // activation scales (fp8 activations)
  int groups, lane, col, c, kgroups_a;
  int tile[4];           // N tile of slot t (clamped into the layer; see tvalid)
  bool tvalid[4];        // slot t holds a real tile
};

// W4A16: bf16 activations, int4/uint4 weights, fp16 group scales (fp32 in the
// packed records), optional zero points. Offset trick: weights enter the MFMA
// as 128+u, the MFMA with the constant -(128+z) (bf16, exact) on the same A
// fragments yields -(128+z)*sum(A) and seeds the accumulation, so the group
// partial is sum A*(q-z) without any per-weight subtraction.
template <bool ASYM>
struct FmtW4A16 {
  using Acc = f32x4_t;
  template <int MT, int NT>
  struct Frag {
    u32x4_t a[MT][4];
    u32x4_t b[NT];
    float s[NT];
    uint32_t o[NT];
  };
  template <int MT, int NT>
  __device__ static void load(Frag<MT, NT>& f, const Ctx& x, int g) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint32_t o = x.aoff[mt] + (uint32_t)(g * 256 + 64 * x.c);
#pragma unroll
      for (int j = 0; j < 4; ++j) f.a[mt][j] = lda(x.arsrc, o + 16 * j);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const size_t u = (size_t)x.tile[t] * x.groups + g;
      f.b[t] = ldg_nt((const u32x4_t*)(x.wbase + u * kUnit4Bytes) + x.lane);
      const u32x2_t r = *((const u32x2_t*)(x.sbase) + u * 16 + x.col);
      f.s[t] = bits_as<float>(r.x);
      f.o[t] = r.y;
    }
  }
  template <int MT, int NT>
  __device__ static void compute(const Frag<MT, NT>& f, Acc (&acc)[MT][NT], uint32_t um, uint32_t ue) {
    f32x4_t corr[MT];
    if constexpr (!ASYM) {
      const u32x4_t k136 = {0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u};  // bf16 -136
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) z = mfma_bf16(f.a[mt][j], k136, z);
        corr[mt] = z;
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      u32x4_t bw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bw[j] = unpack_u4_bf16_offset128(f.b[t][j], um, ue);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4_t p;
        if constexpr (ASYM) {
          const u32x4_t ko = {f.o[t], f.o[t], f.o[t], f.o[t]};
          p = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < 4; ++j) p = mfma_bf16(f.a[mt][j], ko, p);
        } else {
          p = corr[mt];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) p = mfma_bf16(f.a[mt][j], bw[j], p);
        const float s = f.s[t];
        acc[mt][t] = f32x4_t{__builtin_fmaf(s, p[0], acc[mt][t][0]), __builtin_fmaf(s, p[1], acc[mt][t][1]),
                             __builtin_fmaf(s, p[2], acc[mt][t][2]), __builtin_fmaf(s, p[3], acc[mt][t][3])};
      }
    }
  }
  __device__ static float value(float v, const GemmArgs&, int, int) { return v; }
  static constexpr bool kIntAcc = false;
};

// W2A16: bf16 activations, 2-bit weights with fp16 group scales and zero
// points (0..3). The offset trick of W4A16 on 512-byte units: lane (c, col)
// holds its 32 K values in two dwords; each field pair is unpacked to the
// bf16 pair 128 + u with one v_and_or_b32 after a shift, and each group's
// chains start from -(128 + z) * sum(A), the row sums taken once per row
// tile and group.
struct FmtW2A16 {
  using Acc = f32x4_t;
  static constexpr bool kIntAcc = false;
  template <int MT, int NT>
  struct Frag {
    u32x4_t a[MT][4];
    u32x2_t b[NT];
    float s[NT];
    uint32_t o[NT];
  };
  template <int MT, int NT>
  __device__ static void load(Frag<MT, NT>& f, const Ctx& x, int g) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint32_t o = x.aoff[mt] + (uint32_t)(g * 256 + 64 * x.c);
#pragma unroll
      for (int j = 0; j < 4; ++j) f.a[mt][j] = lda(x.arsrc, o + 16 * j);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const size_t u = (size_t)x.tile[t] * x.groups + g;
      f.b[t] = ldg_nt((const u32x2_t*)(x.wbase + u * kUnit2Bytes) + x.lane);
      const u32x2_t r = *((const u32x2_t*)(x.sbase) + u * 16 + x.col);
      f.s[t] = bits_as<float>(r.x);
      f.o[t] = r.y;
    }
  }
  template <int MT, int NT>
  __device__ static void compute(const Frag<MT, NT>& f, Acc (&acc)[MT][NT], uint32_t, uint32_t ue) {
    uint32_t m2;
    asm volatile("v_mov_b32 %0, %1" : "=v"(m2) : "s"(0x00030003u));
    // the group's row sums of A, once per row tile (MFMAs against bf16 1.0):
    // each tile's chains then start from -(128 + z) * rowsum, a multiply
    // instead of four more MFMAs per tile
    f32x4_t rs[MT];
    const u32x4_t one = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) z = mfma_bf16(f.a[mt][j], one, z);
      rs[mt] = z;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      u32x4_t bw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t xw = f.b[t][j / 2];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t v = (xw >> (2 * (4 * (j % 2) + m))) & m2;
          bw[j][m] = v | ue;
        }
      }
      const float negz = __builtin_bit_cast(float, (f.o[t] & 0xFFFFu) << 16);  // -(128+z)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4_t p = {negz * rs[mt][0], negz * rs[mt][1], negz * rs[mt][2], negz * rs[mt][3]};
#pragma unroll
        for (int j = 0; j < 4; ++j) p = mfma_bf16(f.a[mt][j], bw[j], p);
        const float s = f.s[t];
        acc[mt][t] = f32x4_t{__builtin_fmaf(s, p[0], acc[mt][t][0]), __builtin_fmaf(s, p[1], acc[mt][t][1]),
                             __builtin_fmaf(s, p[2], acc[mt][t][2]), __builtin_fmaf(s, p[3], acc[mt][t][3])};
      }
    }
  }
};

// Int8 activations (per token) with int8 (W8A8) or int4 (W4A8) weights.
template <bool W4, bool RAW>
struct FmtInt8 {
  // W8A8 and raw mode accumulate exact int32 over the whole K range; W4A8
  // with scales accumulates fp32 sum_g s_g * P_g with exact int32 P_g.
  static constexpr bool kIntAcc = RAW || !W4;
  using Acc = typename std::conditional<kIntAcc, i32x4_t, f32x4_t>::type;
  template <int MT, int NT>
  struct Frag {
    u32x4_t a[MT][2];
    u32x4_t b[NT][W4 ? 1 : 2];
    float s[NT];
  };
  template <int MT, int NT>
  __device__ static void load(Frag<MT, NT>& f, const Ctx& x, int g) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint32_t o = x.aoff[mt] + (uint32_t)(g * 128 + 32 * x.c);
#pragma unroll
      for (int j = 0; j < 2; ++j) f.a[mt][j] = lda(x.arsrc, o + 16 * j);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const size_t u = (size_t)x.tile[t] * x.groups + g;
      if constexpr (W4) {
        f.b[t][0] = ldg_nt((const u32x4_t*)(x.wbase + u * kUnit4Bytes) + x.lane);
        f.s[t] = RAW ? 0.f : *((const float*)x.sbase + u * 16 + x.col);
      } else {
        const u32x4_t* pu = (const u32x4_t*)(x.wbase + u * kUnit8Bytes);
        f.b[t][0] = ldg_nt(pu + x.lane);
        f.b[t][1] = ldg_nt(pu + 64 + x.lane);
        f.s[t] = 0.f;
      }
    }
  }
  template <int MT, int NT>
  __device__ static void compute(const Frag<MT, NT>& f, Acc (&acc)[MT][NT], uint32_t um, uint32_t ue) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      u32x4_t b0, b1;
      if constexpr (W4) {
        const u32x2_t l0 = unpack_i4_i8x16(f.b[t][0].x), h0 = unpack_i4_i8x16(f.b[t][0].y);
        const u32x2_t l1 = unpack_i4_i8x16(f.b[t][0].z), h1 = unpack_i4_i8x16(f.b[t][0].w);
        b0 = u32x4_t{l0.x, l0.y, h0.x, h0.y};
        b1 = u32x4_t{l1.x, l1.y, h1.x, h1.y};
      } else {
        b0 = f.b[t][0];
        b1 = f.b[t][1];
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if constexpr (kIntAcc) {
          acc[mt][t] = mfma_i8(f.a[mt][1], b1, mfma_i8(f.a[mt][0], b0, acc[mt][t]));
        } else {
          const i32x4_t p = mfma_i8(f.a[mt][1], b1, mfma_i8(f.a[mt][0], b0, i32x4_t{0, 0, 0, 0}));
          const float s = f.s[t];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mt][t][i] = __builtin_fmaf(s, (float)p[i], acc[mt][t][i]);
        }
      }
    }
  }
};

// FP8 E4M3 activations (fp32 scale per token and 128-group) x MXFP4 weights
// (E2M1 with E8M0 block-32 scales applied by the scaled MFMA).
struct FmtMxfp4 {
  using Acc = f32x4_t;
  static constexpr bool kIntAcc = false;
  template <int MT, int NT>
  struct Frag {
    u32x4_t a[MT][2];
    float as[MT][4];
    u32x4_t b[NT];
    uint32_t sc[NT];
  };
  template <int MT, int NT>
  __device__ static void load(Frag<MT, NT>& f, const Ctx& x, int g) {
    // the fp8 operand of the 16x16x128 scaled MFMA is split in two K halves:
    // lane group c holds K 16c..16c+15 (bytes 0-15) and 64+16c..64+16c+15
    // (bytes 16-31); the fp4 operand holds K 32c..32c+31 contiguously
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint32_t o = x.aoff[mt] + (uint32_t)(g * 128 + 16 * x.c);
      f.a[mt][0] = lda(x.arsrc, o);
      f.a[mt][1] = lda(x.arsrc, o + 64);
    }
    // activation scales of the D rows this lane holds: rows 4c+i of each tile
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) f.as[mt][i] = x.a_scales[(size_t)x.as_row[mt][i] * x.groups + g];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const size_t u = (size_t)x.tile[t] * x.groups + g;
      f.b[t] = ldg_nt((const u32x4_t*)(x.wbase + u * kUnit4Bytes) + x.lane);
      f.sc[t] = x.sbase[u * 64 + x.lane];
    }
  }
  template <int MT, int NT>
  __device__ static void compute(const Frag<MT, NT>& f, Acc (&acc)[MT][NT], uint32_t um, uint32_t ue) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const i32x8_t b = {(int)f.b[t].x, (int)f.b[t].y, (int)f.b[t].z, (int)f.b[t].w, 0, 0, 0, 0};
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const i32x8_t a = {(int)f.a[mt][0].x, (int)f.a[mt][0].y, (int)f.a[mt][0].z, (int)f.a[mt][0].w,
                           (int)f.a[mt][1].x, (int)f.a[mt][1].y, (int)f.a[mt][1].z, (int)f.a[mt][1].w};
        const f32x4_t p = mfma_fp8_fp4_scaled(a, b, f32x4_t{0.f, 0.f, 0.f, 0.f}, 127, (int)f.sc[t]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mt][t][i] = __builtin_fmaf(f.as[mt][i], p[i], acc[mt][t][i]);
      }
    }
  }
};

// Per-token int8 activations x MXFP4 weights (the MXFP4 -> INT8 path). The
// fp4 weights stay as they are and go through the same scaled MFMA as the fp8
// path; each int8 activation q is split exactly into q = 16 hi + lo with
// hi in [-8, 7] and lo in [0, 15], both small integers and so exact E4M3
// codes, which a pre-pass writes as two planes (per 128-wide group: 128 hi
// bytes, then 128 lo bytes). A K group is two scaled MFMAs per tile on the
// same weights, the hi plane with the A-scale exponent 2^4: every product is
// exact, the sums are fp32, and the token scale is applied once at the end.
struct FmtMxfp4I8 {
  using Acc = f32x4_t;
  static constexpr bool kIntAcc = false;
  template <int MT, int NT>
  struct Frag {
    u32x4_t a[MT][4];  // hi plane (two K halves), then lo plane
    u32x4_t b[NT];
    uint32_t sc[NT];
  };
  template <int MT, int NT>
  __device__ static void load(Frag<MT, NT>& f, const Ctx& x, int g) {
    // each plane as the fp8 operand of the fp8 path: lane group c holds K
    // 16c..16c+15 and 64+16c..64+16c+15 of the group
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint32_t o = x.aoff[mt] + (uint32_t)(g * 256 + 16 * x.c);
      f.a[mt][0] = lda(x.arsrc, o);
      f.a[mt][1] = lda(x.arsrc, o + 64);
      f.a[mt][2] = lda(x.arsrc, o + 128);
      f.a[mt][3] = lda(x.arsrc, o + 192);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const size_t u = (size_t)x.tile[t] * x.groups + g;
      f.b[t] = ldg_nt((const u32x4_t*)(x.wbase + u * kUnit4Bytes) + x.lane);
      f.sc[t] = x.sbase[u * 64 + x.lane];
    }
  }
  template <int MT, int NT>
  __device__ static void compute(const Frag<MT, NT>& f, Acc (&acc)[MT][NT], uint32_t, uint32_t) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const i32x8_t b = {(int)f.b[t].x, (int)f.b[t].y, (int)f.b[t].z, (int)f.b[t].w, 0, 0, 0, 0};
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4_t h0 = f.a[mt][0], h1 = f.a[mt][1], l0 = f.a[mt][2], l1 = f.a[mt][3];
        const i32x8_t ah = {(int)h0.x, (int)h0.y, (int)h0.z, (int)h0.w, (int)h1.x, (int)h1.y, (int)h1.z, (int)h1.w};
        const i32x8_t al = {(int)l0.x, (int)l0.y, (int)l0.z, (int)l0.w, (int)l1.x, (int)l1.y, (int)l1.z, (int)l1.w};
        acc[mt][t] = mfma_fp8_fp4_scaled(ah, b, acc[mt][t], 127 + 4, (int)f.sc[t]);
        acc[mt][t] = mfma_fp8_fp4_scaled(al, b, acc[mt][t], 127, (int)f.sc[t]);
      }
    }
  }
};

// MXFP4 activations x MXFP4 weights (W4A4): both operands E2M1 with E8M0
// block-32 scales. The scaled MFMA applies both scales exactly, so a K group
// is one MFMA per tile accumulating straight into the fp32 accumulator, with
// no per-group epilogue.
struct FmtW4A4 {
  using Acc = f32x4_t;
  static constexpr bool kIntAcc = false;
  template <int MT, int NT>
  struct Frag {
    u32x4_t a[MT];
    uint32_t as[MT];
    u32x4_t b[NT];
    uint32_t sc[NT];
  };
  template <int MT, int NT>
  __device__ static void load(Frag<MT, NT>& f, const Ctx& x, int g) {
    // lane group c: K 32c..32c+31 of the lane's row (16 bytes of codes) and
    // the E8M0 byte of that block
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f.a[mt] = lda(x.arsrc, x.aoff[mt] + (uint32_t)(g * 64 + 16 * x.c));
      f.as[mt] = x.a_e8m0[(size_t)x.arow_s[mt] * (x.groups * 4) + g * 4 + x.c];
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const size_t u = (size_t)x.tile[t] * x.groups + g;
      f.b[t] = ldg_nt((const u32x4_t*)(x.wbase + u * kUnit4Bytes) + x.lane);
      f.sc[t] = x.sbase[u * 64 + x.lane];
    }
  }
  template <int MT, int NT>
  __device__ static void compute(const Frag<MT, NT>& f, Acc (&acc)[MT][NT], uint32_t, uint32_t) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const i32x8_t b = {(int)f.b[t].x, (int)f.b[t].y, (int)f.b[t].z, (int)f.b[t].w, 0, 0, 0, 0};
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const i32x8_t a = {(int)f.a[mt].x, (int)f.a[mt].y, (int)f.a[mt].z, (int)f.a[mt].w, 0, 0, 0, 0};
        acc[mt][t] = mfma_fp4_fp4_scaled(a, b, acc[mt][t], (int)f.as[mt], (int)f.sc[t]);
      }
    }
  }
};

// W8A16: bf16 activations, int8 weights with one fp32 scale per output
// channel. The weight unit is the W8A8 one (lane group c holds K 32c..32c+15
// in its first 16-byte chunk and 32c+16..32c+31 in its second). Each int8 q
// enters the bf16 MFMA as the integer q + 128 (0..255, exact in bf16: byte to
// fp32 conversion, then the fp32 bits' upper half); a group's chain starts
// from -128 * rowsum(A), so the MFMA sums are exactly sum A*q per group in
// fp32; the channel scale is applied once in the epilogue.
struct FmtW8A16 {
  using Acc = f32x4_t;
  static constexpr bool kIntAcc = false;
  template <int MT, int NT>
  struct Frag {
    u32x4_t a[MT][4];
    u32x4_t b[NT][2];
  };
  template <int MT, int NT>
  __device__ static void load(Frag<MT, NT>& f, const Ctx& x, int g) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint32_t o = x.aoff[mt] + (uint32_t)(g * 256 + 64 * x.c);
#pragma unroll
      for (int j = 0; j < 4; ++j) f.a[mt][j] = lda(x.arsrc, o + 16 * j);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const u32x4_t* pu = (const u32x4_t*)(x.wbase + ((size_t)x.tile[t] * x.groups + g) * kUnit8Bytes);
      f.b[t][0] = ldg_nt(pu + x.lane);
      f.b[t][1] = ldg_nt(pu + 64 + x.lane);
    }
  }
  template <int MT, int NT>
  __device__ static void compute(const Frag<MT, NT>& f, Acc (&acc)[MT][NT], uint32_t, uint32_t) {
    f32x4_t corr[MT];
    const u32x4_t k128 = {0xC300C300u, 0xC300C300u, 0xC300C300u, 0xC300C300u};  // bf16 -128
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) z = mfma_bf16(f.a[mt][j], k128, z);
      corr[mt] = z;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      u32x4_t bw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // step j: K 32c + 8j .. +7 = bytes 8 (j % 2) .. +7 of chunk j / 2
        const u32x4_t ch = f.b[t][j / 2];
        bw[j] = i8x8_bf16_offset128((j % 2) ? ch.z : ch.x, (j % 2) ? ch.w : ch.y);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4_t p = corr[mt];
#pragma unroll
        for (int j = 0; j < 4; ++j) p = mfma_bf16(f.a[mt][j], bw[j], p);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mt][t][i] += p[i];
      }
    }
  }
};

// W4A16-NVFP4: bf16 activations, E2M1 weights with an E4M3 scale per 16 K
// and one binary32 scale per tensor. An E2M1 value (at most 2 significant
// bits) times an E4M3 scale (at most 4 significant bits, exponents -9..8) is
// exact in bf16, so each weight is converted to fp32 by the hardware,
// multiplied by its block scale in fp32 (exact) and packed to bf16 (exact:
// the dropped half is zero). The MFMA then accumulates already-scaled
// products over the whole K range; the tensor scale multiplies the fp32
// result once. The weight unit is the MXFP4 one (lane group c holds K
// 32c..32c+31 of its column, dword j = K 32c+8j..+7, so steps 0-1 use the
// 16-block 2c and steps 2-3 the block 2c+1) and the A fragments are the
// W4A16 ones (the same K values per lane and step).
struct FmtNvfp4 {
  using Acc = f32x4_t;
  static constexpr bool kIntAcc = false;
  template <int MT, int NT>
  struct Frag {
    u32x4_t a[MT][4];
    u32x4_t b[NT];
    uint32_t sc[NT];
  };
  static constexpr int kRecOffset = 256;  // the tensor scale comes first
  template <int MT, int NT>
  __device__ static void load(Frag<MT, NT>& f, const Ctx& x, int g) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint32_t o = x.aoff[mt] + (uint32_t)(g * 256 + 64 * x.c);
#pragma unroll
      for (int j = 0; j < 4; ++j) f.a[mt][j] = lda(x.arsrc, o + 16 * j);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const size_t u = (size_t)x.tile[t] * x.groups + g;
      f.b[t] = ldg_nt((const u32x4_t*)(x.wbase + u * kUnit4Bytes) + x.lane);
      f.sc[t] = ((const uint16_t*)(x.sbase + kRecOffset))[u * 64 + x.lane];
    }
  }
  template <int MT, int NT>
  __device__ static void compute(const Frag<MT, NT>& f, Acc (&acc)[MT][NT], uint32_t, uint32_t) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float s0 = e4m3_to_f32(f.sc[t] & 0xFFu), s1 = e4m3_to_f32((f.sc[t] >> 8) & 0xFFu);
      u32x4_t bw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bw[j] = e2m1x8_scaled_bf16(f.b[t][j], j < 2 ? s0 : s1);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[mt][t] = mfma_bf16(f.a[mt][j], bw[j], acc[mt][t]);
    }
  }
};

// ----------------------------------------------------------------- kernel

template <class F, int MT, int NT, int KW, int U, bool MOE>
__global__ __launch_bounds__(64 * KW) __attribute__((amdgpu_waves_per_eu(MT * NT <= 4 ? 2 : 1))) void stream_gemm_kernel(const GemmArgs p) {
  using Acc = typename F::Acc;
  using Frag = typename F::template Frag<MT, NT>;
  // `wave` must be wave-uniform (an SGPR): every guard around an MFMA has to
  // be a scalar branch, because MFMA instructions ignore the EXEC mask and a
  // lane-masked region would still accumulate whatever the registers hold.
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nb = blockIdx.x, split = blockIdx.y, mb = blockIdx.z;
  constexpr int BM = 16 * MT;
  Ctx x;
  x.lane = lane;
  x.col = lane & 15;
  x.c = lane >> 4;
  x.groups = p.groups;
  // SiLU*mul epilogue (NT = 2): the gate tile nb and the up tile nb + I/16
  const bool silu = p.epi == QDG_EPI_SILU_MUL;
  // Slot t of the workgroup holds N tile nb * NT + t; with the SiLU*mul
  // epilogue slots t < NT/2 hold gate tiles nb * NT/2 + t and slots NT/2 + t
  // the matching up tiles, G = ntiles / 2 further on. Slots past the layer
  // re-read its last tile (every path issues the same loads) and are never
  // stored.
  constexpr int TP = NT > 1 ? NT / 2 : 1;
  const int G = p.ntiles / 2;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (silu) {
      const int j = nb * TP + t % TP;
      x.tvalid[t] = j < G;
      x.tile[t] = (j < G ? j : G - 1) + (t / TP) * G;
    } else {
      const int j = nb * NT + t;
      x.tvalid[t] = j < p.ntiles;
      x.tile[t] = j < p.ntiles ? j : p.ntiles - 1;
    }
  }
  int expert = 0;
  if constexpr (MOE) {
    if (mb * BM >= *p.num_padded) return;
    expert = p.block_expert[mb];
  }
  x.wbase = p.packed + (size_t)expert * p.expert_stride;
  x.sbase = x.wbase + p.s_offset;
  constexpr bool kBf16A = std::is_same<F, FmtW4A16<false>>::value || std::is_same<F, FmtW4A16<true>>::value ||
                          std::is_same<F, FmtW8A16>::value || std::is_same<F, FmtNvfp4>::value ||
                          std::is_same<F, FmtW2A16>::value;
  constexpr bool kFp4A = std::is_same<F, FmtW4A4>::value;
  constexpr bool kPlanesA = std::is_same<F, FmtMxfp4I8>::value;  // two E4M3 planes per row
  const size_t a_row_bytes = kBf16A || kPlanesA ? (size_t)p.K * 2 : kFp4A ? (size_t)p.K / 2 : (size_t)p.K;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = mb * BM + mt * 16 + x.col;
    uint32_t off = kAOob;
    int srow = 0;
    if constexpr (MOE) {
      const int id = p.sorted_ids[r];
      if (id < p.num_pairs) {
        srow = p.a_per_pair ? id : id / p.top_k;
        off = (uint32_t)((size_t)srow * a_row_bytes);
      }
    } else {
      if (r < p.M) {
        srow = r;
        off = (uint32_t)((size_t)r * a_row_bytes);
      }
    }
    x.aoff[mt] = off;
    x.arow_s[mt] = srow;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int rr = mb * BM + mt * 16 + 4 * x.c + ii;
      int srr = 0;
      if constexpr (MOE) {
        const int id = p.sorted_ids[rr];
        srr = id < p.num_pairs ? (p.a_per_pair ? id : id / p.top_k) : 0;
      } else {
        srr = rr < p.M ? rr : 0;
      }
      x.as_row[mt][ii] = srr;
    }
  }
  x.a_scales = p.a_scales;
  x.a_e8m0 = (const uint8_t*)p.a_scales;
  x.arsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p.A), (short)0, (int)p.a_bytes, 0x00020000);

  const int g0 = (int)(((int64_t)split * p.groups) / p.split);
  const int g1 = (int)(((int64_t)(split + 1) * p.groups) / p.split);
  const int cnt = (g1 - g0 - wave + KW - 1) / KW;  // groups of this wave

  Acc acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[mt][t] = Acc{0, 0, 0, 0};

  Frag fa[U], fb[U];
  // Every chunk issues the same loads on every path (groups past this wave's
  // last one re-read that group), so the compiler's load waits stay exact and
  // the next chunk's loads remain in flight while the current one computes;
  // a conditional load would make every wait a wait for all loads.
  auto load_chunk = [&](Frag(&f)[U], int i) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int gi = i + u < cnt ? i + u : cnt - 1;
      F::template load<MT, NT>(f[u], x, g0 + wave + KW * gi);
    }
  };
  // W4A16 unpack constants in registers (a VGPR mask and a scalar exponent):
  // each unpacked dword is then one v_and_or_b32 (VOP3 takes no literals)
  uint32_t um;
  asm volatile("v_mov_b32 %0, %1" : "=v"(um) : "s"(0x000F000Fu));
  const uint32_t ue = 0x43004300u;
  auto compute_full = [&](const Frag(&f)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) F::template compute<MT, NT>(f[u], acc, um, ue);
  };
  auto compute_chunk = [&](const Frag(&f)[U], int i) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i + u < cnt) F::template compute<MT, NT>(f[u], acc, um, ue);
  };
  if (cnt > 0) {
    load_chunk(fa, 0);
    int i = 0;
    for (; i + 2 * U < cnt; i += 2 * U) {  // chunks i, i + U complete; chunk i + 2U started
      load_chunk(fb, i + U);
      compute_full(fa);
      load_chunk(fa, i + 2 * U);
      compute_full(fb);
    }
    if (i + U < cnt) {
      load_chunk(fb, i + U);
      compute_full(fa);
      compute_chunk(fb, i + U);
    } else {
      compute_chunk(fa, i);
    }
  }

  // ---- reduce the KW wave partials through LDS (fixed order: wave 0 + 1 + ...)
  constexpr int kVals = MT * NT * 4;
  __shared__ float red[(KW > 1 ? KW - 1 : 1) * kVals * 64];
  if constexpr (KW > 1) {
    if (wave > 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            red[(((wave - 1) * MT + mt) * NT * 4 + t * 4 + i) * 64 + lane] =
                bits_as<float>(acc[mt][t][i]);
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 1; w < KW; ++w)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = red[(((w - 1) * MT + mt) * NT * 4 + t * 4 + i) * 64 + lane];
            if constexpr (F::kIntAcc)
              acc[mt][t][i] += __builtin_bit_cast(int, v);
            else
              acc[mt][t][i] += v;
          }
  }

  // ---- split-K (dense, not raw int32): the scaled fp32 partial of this
  // split goes to the workspace as [split][m_pad][n_pad], and
  // reduce_splits_kernel adds the splits in split order (deterministic; no
  // cross-workgroup fences, which on this part write back and invalidate L2)
  const bool to_partial = p.split > 1;
  const int n_pad = gridDim.x * NT * 16;

  // ---- epilogue: final scaling and store
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = mb * BM + mt * 16 + 4 * x.c + i;
      int yrow = r, arow = r;
      bool v;
      if constexpr (MOE) {
        const int id = p.sorted_ids[r];
        v = id < p.num_pairs;
        yrow = id;
        arow = v ? (p.a_per_pair ? id : id / p.top_k) : 0;
      } else {
        v = r < p.M;
      }
      if (!v) continue;
      float yv[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int n = x.tile[t] * 16 + x.col;
        yv[t] = 0.f;
        if (!x.tvalid[t] || n >= p.N) continue;
        const size_t o = (size_t)yrow * p.N + n;
        if (p.otype == QDG_O_I32) {
          int v = bits_as<int>(acc[mt][t][i]);
          // W4A8 accumulates 16*q*qa (int4 moved to the high nibble): exact shift back
          if constexpr (std::is_same<F, FmtInt8<true, true>>::value) v >>= 4;
          ((int*)p.Y)[o] = v;
          continue;
        }
        float y;
        if constexpr (std::is_same<F, FmtInt8<false, false>>::value) {
          // W8A8: exact int32 sum, then per-token x per-channel scale
          const float sw = ((const float*)x.sbase)[n];
          y = (float)acc[mt][t][i] * p.a_scales[arow] * sw;
        } else if constexpr (std::is_same<F, FmtW8A16>::value) {
          y = acc[mt][t][i] * ((const float*)x.sbase)[n];  // per-channel scale
        } else if constexpr (std::is_same<F, FmtNvfp4>::value) {
          y = acc[mt][t][i] * ((const float*)x.sbase)[0];  // tensor scale
        } else if constexpr (std::is_same<F, FmtInt8<true, false>>::value || std::is_same<F, FmtMxfp4I8>::value) {
          y = acc[mt][t][i] * p.a_scales[arow];  // per-token activation scale
        } else if constexpr (F::kIntAcc) {
          y = (float)acc[mt][t][i];
        } else {
          y = acc[mt][t][i];
        }
        yv[t] = y;
        if (to_partial) {
          ((float*)p.partial)[((size_t)split * p.m_pad + r) * n_pad + n] = y;
          continue;
        }
        if (silu) continue;
        if (p.otype == QDG_O_F32)
          ((float*)p.Y)[o] = y;
        else
          ((uint16_t*)p.Y)[o] = (uint16_t)f32_to_bf16_rne(y);
      }
      if (silu) {
        // gate in slot t, up in slot t + NT/2; Y rows hold I = N / 2 columns
#pragma unroll
        for (int t = 0; t < TP; ++t) {
          if (!x.tvalid[t]) continue;
          const float g = yv[t], u = yv[t + TP];
          const float h = g / (1.f + expf(-g)) * u;
          const size_t o = (size_t)yrow * (p.N / 2) + (nb * TP + t) * 16 + x.col;
          if (p.otype == QDG_O_F32)
            ((float*)p.Y)[o] = h;
          else
            ((uint16_t*)p.Y)[o] = (uint16_t)f32_to_bf16_rne(h);
        }
      }
    }
  }
}

#ifndef __HIPCC_RTC__  // host launchers
template <class F, int MT, int NT, int KW, int U>
hipError_t launch_one(bool moe, const GemmArgs& a, int grid_m, hipStream_t s) {
  dim3 grid((a.ntiles + NT - 1) / NT, a.split, grid_m);
  dim3 block(64 * KW);
  if (moe)
    hipLaunchKernelGGL((stream_gemm_kernel<F, MT, NT, KW, U, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((stream_gemm_kernel<F, MT, NT, KW, U, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <class F>
hipError_t dispatch_shape(const StreamCfg& c, bool moe, const GemmArgs& a, int grid_m, hipStream_t s) {
#define QDG_CASE(MT_, NT_, KW_)                                       \
  if (c.mt == MT_ && c.nt == NT_ && c.kw == KW_)                      \
    return launch_one<F, MT_, NT_, KW_, 2>(moe, a, grid_m, s);
  QDG_CASE(1, 1, 4)
  QDG_CASE(1, 2, 4)
  QDG_CASE(1, 4, 4)
  QDG_CASE(2, 2, 4)
  QDG_CASE(2, 4, 4)
  QDG_CASE(4, 2, 4)
  QDG_CASE(4, 4, 4)
#undef QDG_CASE
  return hipErrorInvalidValue;
}

#endif
}  // namespace

#ifndef __HIPCC_RTC__  // host launchers
bool stream_cfg_supported(Format, const StreamCfg& c) {
  if (c.kw != 4) return false;
  if (c.mt == 1) return c.nt == 1 || c.nt == 2 || c.nt == 4;
  if (c.mt == 2 || c.mt == 4) return c.nt == 2 || c.nt == 4;
  return false;
}

hipError_t launch_stream(Format f, bool asym, bool moe, const StreamCfg& c, const GemmArgs& a,
                         int grid_m, hipStream_t s) {
  const bool raw = a.otype == QDG_O_I32;
  switch (f) {
    case FMT_W4A16:
      return asym ? dispatch_shape<FmtW4A16<true>>(c, moe, a, grid_m, s)
                  : dispatch_shape<FmtW4A16<false>>(c, moe, a, grid_m, s);
    case FMT_W8A8:
      return raw ? dispatch_shape<FmtInt8<false, true>>(c, moe, a, grid_m, s)
                 : dispatch_shape<FmtInt8<false, false>>(c, moe, a, grid_m, s);
    case FMT_W4A8:
      return raw ? dispatch_shape<FmtInt8<true, true>>(c, moe, a, grid_m, s)
                 : dispatch_shape<FmtInt8<true, false>>(c, moe, a, grid_m, s);
    case FMT_MXFP4:
      return dispatch_shape<FmtMxfp4>(c, moe, a, grid_m, s);
    case FMT_W4A4:
      return dispatch_shape<FmtW4A4>(c, moe, a, grid_m, s);
    case FMT_MXFP4_I8:
      return dispatch_shape<FmtMxfp4I8>(c, moe, a, grid_m, s);
    case FMT_W2A16:
      return dispatch_shape<FmtW2A16>(c, moe, a, grid_m, s);
    case FMT_W8A16:
      return dispatch_shape<FmtW8A16>(c, moe, a, grid_m, s);
    case FMT_NVFP4:
      return dispatch_shape<FmtNvfp4>(c, moe, a, grid_m, s);
  }
  return hipErrorInvalidValue;
}

#endif

}  // namespace qdg
