// Activation quantization for the integer and fp8 paths (bf16 in).
//
// The pages name W8A8 and W4A8 as common configurations (kinachrichten,
// "Warum quantisierte Kernel wichtig sind"; jetabc, section on what
// quantization is) without the activation scheme. Implemented schemes:
//   int8, one fp32 scale per token:   inv = f32(127/amax), q = rne(clamp(x*inv))
//   fp8 E4M3 (OCP), one fp32 scale per token and 128-wide K group:
//                                     inv = f32(448/amax), q = e4m3_rne(clamp(x*inv))
//   MXFP4 (OCP MX), one E8M0 scale per token and 32-wide K block:
//                                     X = floor(log2(amax)) - 2, q = e2m1_rne_sat(x / 2^X)
// Scale = f32(amax/Q); amax = 0 gives scale 1 and zero codes. Every step is
// binary32 with RNE and correctly rounded division, so the codes are
// reproducible bit for bit by any implementation doing the same steps. The
// E4M3 and E2M1 encodes run on gfx950's conversion instructions
// (v_cvt_pk_fp8_f32, v_cvt_scalef32_pk_fp4_f32: round to nearest even, the
// sign kept on zero); the tests compare them with the oracle's encoders over
// every bf16 input magnitude the encodes can see.
#include "qdg_device.h"
#include "qdg_internal.h"

namespace qdg {
namespace {

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __builtin_bit_cast(float, h << 16); }


// MXFP4 per (token, 32-block): four lanes per block, 8 values (16 bytes) each;
// the block's amax comes from a 4-lane reduction. X is read from the
// exponent field of amax (a subnormal amax, below 2^-126, gives the clamped
// X = -127), and x / 2^X is a product with the power of two 2^-X, exact for
// every value whose code is not 0.
__global__ __launch_bounds__(256) void act_fp4_kernel(const uint16_t* __restrict__ a, uint8_t* __restrict__ q,
                                                      uint8_t* __restrict__ scales, int64_t blocks) {
  const int64_t gl = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t b = gl >> 2;  // block index: row * (K/32) + j
  const int sub = threadIdx.x & 3;
  if (b >= blocks) return;    // whole 4-lane segments exit together
  const u32x4_t v = *(const u32x4_t*)(a + b * 32 + sub * 8);
  float f[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = bf16_to_f32(v[j] & 0xFFFFu);
    f[2 * j + 1] = bf16_to_f32(v[j] >> 16);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 4));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 4));
  uint32_t out = 0, e8 = 0;
  if (amax > 0.f) {
    const int ef = (int)((__builtin_bit_cast(uint32_t, amax) >> 23) & 0xFFu);
    int X = ef == 0 ? -127 : ef - 127 - 2;  // floor(log2(amax)) - 2
    X = X < -127 ? -127 : X;
    e8 = (uint32_t)(X + 127);
    const float inv = __builtin_bit_cast(float, (uint32_t)(127 - X) << 23);  // 2^-X, X in [-127, 125]
    // gfx950's v_cvt_scalef32_pk_fp4_f32 encodes two binary32 values as
    // E2M1 with round to nearest even and saturation at +-6 (sign kept for
    // values that round to zero); with scale 1 it encodes x / 2^X itself,
    // element 2j in the low nibble of byte j
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, f[0] * inv, f[1] * inv, 1.0f, 0);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, f[2] * inv, f[3] * inv, 1.0f, 1);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, f[4] * inv, f[5] * inv, 1.0f, 2);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, f[6] * inv, f[7] * inv, 1.0f, 3);
  }
  *(uint32_t*)(q + b * 16 + sub * 4) = out;
  if (sub == 0) scales[b] = (uint8_t)e8;
}

// int8 per token: one workgroup per row.
__global__ __launch_bounds__(256) void act_int8_kernel(const uint16_t* __restrict__ a, int8_t* __restrict__ q,
                                                       float* __restrict__ scales, int64_t K) {
  const int64_t row = blockIdx.x;
  const uint16_t* x = a + row * K;
  float amax = 0.f;
  for (int64_t k = threadIdx.x * 8; k < K; k += 256 * 8) {
    const u32x4_t v = *(const u32x4_t*)(x + k);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      amax = fmaxf(amax, fabsf(bf16_to_f32(v[i] & 0xFFFFu)));
      amax = fmaxf(amax, fabsf(bf16_to_f32(v[i] >> 16)));
    }
  }
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  __shared__ float wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const bool nz = amax > 0.f;
  const float inv = nz ? __fdiv_rn(127.0f, amax) : 0.f;
  if (threadIdx.x == 0) scales[row] = nz ? __fdiv_rn(amax, 127.0f) : 1.0f;
  int8_t* y = q + row * K;
  for (int64_t k = threadIdx.x * 8; k < K; k += 256 * 8) {
    const u32x4_t v = *(const u32x4_t*)(x + k);
    u32x2_t out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float f0 = fminf(fmaxf(rintf(bf16_to_f32(v[i] & 0xFFFFu) * inv), -127.f), 127.f);
      const float f1 = fminf(fmaxf(rintf(bf16_to_f32(v[i] >> 16) * inv), -127.f), 127.f);
      const uint32_t b = ((uint32_t)(int)f0 & 0xFFu) | (((uint32_t)(int)f1 & 0xFFu) << 8);
      if (i & 1) out[i >> 1] |= b << 16;
      else out[i >> 1] = b;
    }
    *(u32x2_t*)(y + k) = out;
  }
}

// fp8 per (token, 128-group): 16 lanes per group, 8 values per lane.
__global__ __launch_bounds__(256) void act_fp8_kernel(const uint16_t* __restrict__ a, uint8_t* __restrict__ q,
                                                      float* __restrict__ scales, int64_t M, int64_t K) {
  const int64_t gid = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;  // (row, group) index
  const int sub = threadIdx.x & 15;
  const int64_t groups = K / 128;
  if (gid >= M * groups) return;  // whole 16-lane segments exit together
  const int64_t row = gid / groups, g = gid % groups;
  const uint16_t* x = a + row * K + g * 128 + sub * 8;
  const u32x4_t v = *(const u32x4_t*)x;
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_to_f32(v[i] & 0xFFFFu);
    f[2 * i + 1] = bf16_to_f32(v[i] >> 16);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  for (int off = 8; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
  const bool nz = amax > 0.f;
  const float inv = nz ? __fdiv_rn(448.0f, amax) : 0.f;
  if (sub == 0) scales[row * groups + g] = nz ? __fdiv_rn(amax, 448.0f) : 1.0f;
  // gfx950's v_cvt_pk_fp8_f32 encodes two binary32 values as OCP E4M3 with
  // round to nearest even (subnormal codes included, the sign kept for
  // values that round to zero); inputs are clamped to the largest finite
  // magnitude first, so no code is NaN
  u32x2_t out = {0, 0};
  if (nz) {
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = fminf(fmaxf(f[i] * inv, -448.f), 448.f);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(t[4 * j], t[4 * j + 1], 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(t[4 * j + 2], t[4 * j + 3], w, true);
      out[j] = (uint32_t)w;
    }
  }
  *(u32x2_t*)(q + row * K + g * 128 + sub * 8) = out;
}

}  // namespace

namespace {

// int8 activation codes -> two E4M3 planes, q = 16 * hi + lo with
// hi = q >> 4 in [-8, 7] and lo = q & 15 in [0, 15]: one thread per 16 codes.
// Both halves are integers that E4M3 holds exactly (at most 4 significant
// bits), so gfx950's v_cvt_pk_fp8_f32 (OCP E4M3, two values per
// instruction) encodes them without rounding.
__global__ __launch_bounds__(256) void act_i8_planes_kernel(const int8_t* __restrict__ qa, int64_t rows, int64_t K,
                                                          uint8_t* __restrict__ planes) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // 16-code chunk
  const int64_t per_row = K / 16;
  if (q >= rows * per_row) return;
  const int64_t r = q / per_row, k0 = (q % per_row) * 16;
  const u32x4_t v = *(const u32x4_t*)(qa + r * K + k0);
  u32x4_t hi, lo;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    float h[4], l[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int code = (int)(int8_t)(v[d] >> (8 * b));
      h[b] = (float)(code >> 4);
      l[b] = (float)(code & 15);
    }
    int wh = __builtin_amdgcn_cvt_pk_fp8_f32(h[0], h[1], 0, false);
    wh = __builtin_amdgcn_cvt_pk_fp8_f32(h[2], h[3], wh, true);
    int wl = __builtin_amdgcn_cvt_pk_fp8_f32(l[0], l[1], 0, false);
    wl = __builtin_amdgcn_cvt_pk_fp8_f32(l[2], l[3], wl, true);
    hi[d] = (uint32_t)wh;
    lo[d] = (uint32_t)wl;
  }
  uint8_t* row = planes + r * 2 * K + (k0 / 128) * 256 + (k0 % 128);
  *(u32x4_t*)row = hi;
  *(u32x4_t*)(row + 128) = lo;
}

}  // namespace

hipError_t launch_act_i8_planes(const int8_t* qa, int64_t rows, int64_t K, uint8_t* planes, hipStream_t s) {
  const int64_t threads = rows * (K / 16);
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(act_i8_planes_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, qa, rows, K,
                     planes);
  return hipGetLastError();
}

hipError_t launch_quantize_act(int atype, const void* a, int64_t M, int64_t K, void* qa, float* scales,
                               hipStream_t s) {
  if (atype == QDG_A_INT8) {
    hipLaunchKernelGGL(act_int8_kernel, dim3((unsigned)M), dim3(256), 0, s, (const uint16_t*)a, (int8_t*)qa,
                       scales, K);
  } else if (atype == QDG_A_MXFP4) {
    const int64_t blocks = M * (K / 32);
    hipLaunchKernelGGL(act_fp4_kernel, dim3((unsigned)((blocks * 4 + 255) / 256)), dim3(256), 0, s,
                       (const uint16_t*)a, (uint8_t*)qa, (uint8_t*)scales, blocks);
  } else {
    const int64_t threads = M * (K / 128) * 16;
    hipLaunchKernelGGL(act_fp8_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                       (const uint16_t*)a, (uint8_t*)qa, scales, M, K);
  }
  return hipGetLastError();
}

}  // namespace qdg
