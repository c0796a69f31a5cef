// Device-side building blocks shared by the gfx950 kernels: vector types,
// MFMA wrappers, unpackers and the packed-layout constants.
//
// The packed layout is organised in "units": 16 output columns x 128 K values
// (one K-group of the group-128 formats). A unit is consumed by one wavefront
// with one (or two) 16-byte loads per lane, so every unit read is a fully
// coalesced 1 KiB (or 2 KiB) access. Lane l of a wave owns column l % 16 and
// the K quarter c = l / 16 (32 consecutive K values) of the unit; the MFMA
// operand of lane l is therefore built from A[row][32c .. 32c+31] and the
// matching weights, which keeps the A loads contiguous as well.
#pragma once
#ifdef __HIPCC_RTC__
// Run-time compilation (hipRTC, qdg_plan_jit) has no C library headers: the
// fixed-width types and the two type traits the kernels use, from the
// compiler's own definitions.
typedef __INT8_TYPE__ int8_t;
typedef __UINT8_TYPE__ uint8_t;
typedef __INT16_TYPE__ int16_t;
typedef __UINT16_TYPE__ uint16_t;
typedef __INT32_TYPE__ int32_t;
typedef __UINT32_TYPE__ uint32_t;
typedef __INT64_TYPE__ int64_t;
typedef __UINT64_TYPE__ uint64_t;
typedef __SIZE_TYPE__ size_t;
typedef __UINTPTR_TYPE__ uintptr_t;
namespace std {
template <class A, class B> struct is_same { static constexpr bool value = false; };
template <class A> struct is_same<A, A> { static constexpr bool value = true; };
template <bool C, class T, class F> struct conditional { using type = T; };
template <class T, class F> struct conditional<false, T, F> { using type = F; };
}  // namespace std
#else
#include <hip/hip_runtime.h>
#include <stdint.h>
#endif

namespace qdg {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

constexpr int kUnitK = 128;      // K values per unit (= group size)
constexpr int kUnitN = 16;       // columns per unit
constexpr int kUnit4Bytes = 1024;  // 4-bit unit
constexpr int kUnit8Bytes = 2048;  // int8 unit
constexpr int kUnit2Bytes = 512;   // 2-bit unit

// ------------------------------------------------------------------ MFMA
// v_mfma_f32_16x16x32_bf16: D[16x16] += A[16x32] B[32x16]. Lane l supplies
// row (A) / column (B) l%16 and 8 K values; D lane l holds column l%16,
// rows 4*(l/16) + i. The K order inside an operand is irrelevant to the
// product as long as A and B use the same one, which the packers ensure.
__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// v_mfma_f32_32x32x16_bf16: D[32x32] += A[32x16] B[16x32]. Lane l supplies
// row (A) / column (B) l%32 and 8 K values (lane half l/32 the second 8 of
// the step); D lane l holds column l%32, rows 8*(i/4) + 4*(l/32) + i%4
// (measured). Twice the work of the 16 x 16 form per issued instruction.
__device__ __forceinline__ f32x16_t mfma_bf16_32(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// v_mfma_i32_16x16x64_i8: 16 int8 per lane, exact int32 accumulation.
__device__ __forceinline__ i32x4_t mfma_i8(u32x4_t a, u32x4_t b, i32x4_t c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4_t, a),
                                               __builtin_bit_cast(i32x4_t, b), c, 0, 0, 0);
}

// v_mfma_scale_f32_16x16x128_f8f6f4 with A = FP8 E4M3 (format 0) and
// B = FP4 E2M1 (format 4); lane l supplies row (A) / column (B) l%16. Measured
// operand layout: the FP4 operand of lane group c = l/16 holds K 32c..32c+31
// in nibble order (4 dwords); the FP8 operand of lane group c holds K
// 16c..16c+15 in bytes 0-15 and K 64+16c..64+16c+15 in bytes 16-31. The E8M0
// scale of lane group c (byte 0 of sa / sb) applies to the K block
// 32c..32c+31 of that lane's row / column.
__device__ __forceinline__ f32x4_t mfma_fp8_fp4_scaled(i32x8_t a, i32x8_t b, f32x4_t c, int sa,
                                                       int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, sa, 0, sb);
}

// The same scaled MFMA with both operands FP4 E2M1 (format 4, W4A4): each
// lane supplies 32 E2M1 values of its row / column (16 bytes, the low four
// dwords; lane group c holds K 32c..32c+31) and the E8M0 byte of that block.
__device__ __forceinline__ f32x4_t mfma_fp4_fp4_scaled(i32x8_t a, i32x8_t b, f32x4_t c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
}

// ------------------------------------------------------------------ unpack
// W4A16: one dword holds 8 biased nibbles u (u = q for uint4, q + 8 for
// int4). Element 2i of the MFMA operand is nibble i, element 2i+1 is nibble
// i+4. Each nibble becomes the bf16 number 128 + u (exponent of 128 with u
// in the low mantissa bits: exact), so the MFMA sees weights offset by 128;
// the offset and the zero point are removed through the row sums of A.
__device__ __forceinline__ u32x4_t unpack_u4_bf16_offset128(uint32_t x) {
  u32x4_t r;
  r.x = (x & 0x000F000Fu) | 0x43004300u;
  r.y = ((x >> 4) & 0x000F000Fu) | 0x43004300u;
  r.z = ((x >> 8) & 0x000F000Fu) | 0x43004300u;
  r.w = ((x >> 12) & 0x000F000Fu) | 0x43004300u;
  return r;
}

// Same as above with the mask and exponent constants held in registers
// (m = 0x000F000F, e = 0x43004300): each output dword is then one
// v_and_or_b32 (plus a shift), since VOP3 forms cannot take literals.
__device__ __forceinline__ u32x4_t unpack_u4_bf16_offset128(uint32_t x, uint32_t m, uint32_t e) {
  u32x4_t r;
  r.x = (x & m) | e;
  r.y = ((x >> 4) & m) | e;
  r.z = ((x >> 8) & m) | e;
  r.w = ((x >> 12) & m) | e;
  return r;
}

// W4A8: two's-complement nibbles moved into the high half of a byte give the
// int8 value 16*q exactly; the factor 16 is folded into the group scale.
// Byte i of the low result is nibble 2i, byte i of the high result nibble 2i+1.
__device__ __forceinline__ u32x2_t unpack_i4_i8x16(uint32_t x) {
  u32x2_t r;
  r.x = (x << 4) & 0xF0F0F0F0u;
  r.y = x & 0xF0F0F0F0u;
  return r;
}

// ------------------------------------------------------------------ misc
// Bit reinterpretation through a by-value scalar. Applying __builtin_bit_cast
// directly to an ext_vector element (v[i]) is miscompiled by this toolchain
// (it reads element 0 for every i), so vector elements always go through
// this function.
template <class To, class From>
__device__ __forceinline__ To bits_as(From v) {
  static_assert(sizeof(To) == sizeof(From), "size mismatch");
  return __builtin_bit_cast(To, v);
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (u >> 16) | 0x40u;  // NaN
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <typename T>
__device__ __forceinline__ T ldg_nt(const T* p) {
  return __builtin_nontemporal_load(p);
}

// OCP E4M3 ("fn") encoding of a finite value with |v| <= 448, RNE; the sign
// of zero is kept. Written from the format definition: bias 7, 3 mantissa
// bits, exponent field 0 subnormal (units of 2^-9).
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t sign = __builtin_signbit(v) ? 0x80u : 0u;
  const float a = fabsf(v);
  const uint32_t u = __builtin_bit_cast(uint32_t, a);
  const int e = (int)(u >> 23) - 127;
  uint32_t code;
  if (e < -6) {
    code = (uint32_t)rintf(a * 512.0f);  // exact scaling; 8 becomes the min normal
  } else {
    const uint32_t mant = u & 0x7FFFFFu;
    uint32_t m = mant >> 20;
    const uint32_t rem = mant & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) ++m;
    int ee = e;
    if (m == 8) {
      m = 0;
      ++ee;
    }
    code = ((uint32_t)(ee + 7) << 3) | m;
  }
  return code | sign;
}

// NVFP4 weights: OCP E4M3 block-scale code -> its exact fp32 value (the NaN
// codes are mapped away by preprocess), and two E2M1 codes (byte SEL of d,
// even k in the low nibble) times that scale -> a bf16 pair. The products are
// exact in bf16 (at most 2 x 4 significant bits, exponents far inside the
// range), so the fp32 multiply is exact and the pack drops only zero bits.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float mag = e ? __builtin_bit_cast(float, ((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (b & 0x80u) ? -mag : mag;
}
template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2_scaled_bf16(uint32_t d, float s) {
  const f32x2_t v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, SEL);
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, v.y * s), __builtin_bit_cast(uint32_t, v.x * s),
                               0x07060302u);
}
// W8A16: four int8 codes (one dword, K order) -> two bf16 pairs of the
// integers q + 128 (0..255, exact: byte -> fp32 conversion, then the fp32
// word's upper half)
__device__ __forceinline__ void widen_i8_bf16_offset128(uint32_t d, uint32_t& lo, uint32_t& hi) {
  const uint32_t u = d ^ 0x80808080u;
  const uint32_t f0 = __builtin_bit_cast(uint32_t, (float)(u & 0xFFu));
  const uint32_t f1 = __builtin_bit_cast(uint32_t, (float)((u >> 8) & 0xFFu));
  const uint32_t f2 = __builtin_bit_cast(uint32_t, (float)((u >> 16) & 0xFFu));
  const uint32_t f3 = __builtin_bit_cast(uint32_t, (float)(u >> 24));
  lo = __builtin_amdgcn_perm(f1, f0, 0x07060302u);
  hi = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
}
// eight int8 codes (two dwords, K order) -> a bf16 MFMA operand of q + 128
__device__ __forceinline__ u32x4_t i8x8_bf16_offset128(uint32_t d0, uint32_t d1) {
  uint32_t w0, w1, w2, w3;
  widen_i8_bf16_offset128(d0, w0, w1);
  widen_i8_bf16_offset128(d1, w2, w3);
  return u32x4_t{w0, w1, w2, w3};
}
// eight E2M1 codes (one dword, K order) times s -> a bf16 MFMA operand
__device__ __forceinline__ u32x4_t e2m1x8_scaled_bf16(uint32_t d, float s) {
  return u32x4_t{e2m1x2_scaled_bf16<0>(d, s), e2m1x2_scaled_bf16<1>(d, s), e2m1x2_scaled_bf16<2>(d, s),
                 e2m1x2_scaled_bf16<3>(d, s)};
}

// Tile order of the LDS-tiled grouped MoE launches. Which expert blocks hold
// rows is known on the device only (the first num_padded / BM of the
// capacity), so the order must not hand any XCD a range of empty blocks:
// workgroup ids go to the 8 XCDs in turn, and id i takes block
// 8 * (i / 8 / n_blocks) + i % 8 and column block (i / 8) % n_blocks. Every
// XCD then runs whole blocks (all their column blocks, so a block's A rows
// stay in that XCD's L2), and on every XCD the blocks that hold rows come
// first. The grid covers whole groups of 8 blocks (moe_grid_blocks); blocks
// past the capacity return like the empty ones.
__device__ __forceinline__ void moe_tile_order(int n_blocks, int& mb, int& nb) {
  const int x = (int)(blockIdx.x % 8u), j = (int)(blockIdx.x / 8u);
  mb = (j / n_blocks) * 8 + x;
  nb = j % n_blocks;
}

__host__ __device__ constexpr int moe_grid_blocks(int m_blocks) { return (m_blocks + 7) / 8 * 8; }

}  // namespace qdg
