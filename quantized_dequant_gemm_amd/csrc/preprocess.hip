// Preprocessing: standard format -> gfx950 kernel layout, and the producer of
// the standard format from float32 weights.
//
// The pages describe a preprocessing step that checks parameters, pads
// dimensions and repacks tensors for the target kernel, and stress that a
// repack rearranges storage without changing the quantization method
// (kinachrichten, "Wie die Architektur funktioniert"; "vLLM Humming: why
// shared quantization still needs specialized kernels", section
// "Representation answers a different question"). Here the repack is a pure
// permutation of nibbles/bytes into 16-column x 128-K units (see
// qdg_device.h) plus per-unit scale records; N is padded to a multiple of 16.
#include "qdg_device.h"
#include "qdg_internal.h"

namespace qdg {
namespace {

__device__ __forceinline__ uint32_t permute_nibbles(uint32_t in, const int (&src)[8]) {
  uint32_t out = 0;
#pragma unroll
  for (int p = 0; p < 8; ++p) out |= ((in >> (4 * src[p])) & 0xFu) << (4 * p);
  return out;
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Sets an input flag in the caller's status word (a vector atomic; taken
// only on bad input, so it costs nothing on the common path).
__device__ __forceinline__ void raise_flag(uint32_t* status, uint32_t flag) {
  if (status) atomicOr(status, flag);
}

__device__ __forceinline__ bool finite_f32(float x) {
  return (__builtin_bit_cast(uint32_t, x) & 0x7F800000u) != 0x7F800000u;
}

// One thread per (expert, tile, group, lane): writes the lane's 16 bytes of
// the unit (32 bytes for int8) and, for lanes 0..15, the scale record of
// column `lane`.
__global__ void repack_kernel(int fmt, int wtype, const uint8_t* __restrict__ qw,
                              const void* __restrict__ scales, const uint8_t* __restrict__ zeros,
                              const float* __restrict__ tscale, uint8_t* __restrict__ packed, int64_t N, int64_t K, int64_t ntiles,
                              int64_t groups, int64_t expert_stride, int64_t s_offset, int64_t experts,
                              uint32_t* __restrict__ status) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_expert = ntiles * groups * 64;
  if (tid >= per_expert * experts) return;
  const int64_t e = tid / per_expert;
  int64_t r = tid % per_expert;
  const int lane = (int)(r & 63);
  r >>= 6;
  const int64_t g = r % groups;
  const int64_t tile = r / groups;
  const int c = lane >> 4, col = lane & 15;
  const int64_t n = tile * 16 + col;
  const bool valid = n < N;
  const int64_t unit = tile * groups + g;
  uint8_t* wdst = packed + e * expert_stride;
  uint8_t* sdst = wdst + s_offset;

  if (fmt == FMT_W2A16) {
    // 512-byte unit: lane (c, col) holds K 32c .. 32c+31 of its column in two
    // dwords; dword d serves the MFMA K steps 2d and 2d+1 (K 32c + 8j .. +7).
    // Field i = 4h + m (h = step within the dword, m = bf16 pair of the
    // operand) sits at bits 2i (element 2m of step 2d+h) and 16 + 2i
    // (element 2m+1), so (x >> 2i) & 0x00030003 | 0x43004300 is that pair as
    // bf16 128 + u.
    const uint8_t* src = qw + (e * N + (valid ? n : 0)) * (K / 4);
    u32x2_t out = {0, 0};
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      uint32_t v = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t k0 = g * 128 + 32 * c + 16 * d + 8 * (i >> 2) + 2 * (i & 3);
        const uint32_t c0 = (src[k0 / 4] >> (2 * (k0 % 4))) & 3u;
        const uint32_t c1 = (src[(k0 + 1) / 4] >> (2 * ((k0 + 1) % 4))) & 3u;
        v |= (c0 << (2 * i)) | (c1 << (16 + 2 * i));
      }
      out[d] = valid ? v : 0u;
    }
    *((u32x2_t*)(wdst + unit * kUnit2Bytes) + lane) = out;
    if (c == 0) {
      const float s = valid ? half_bits_to_float(((const uint16_t*)scales)[(e * N + n) * groups + g]) : 0.f;
      if (!finite_f32(s)) raise_flag(status, QDG_FLAG_BAD_SCALE);
      const uint32_t zq = valid ? zeros[(e * N + n) * groups + g] : 0;
      if (zq > 3) raise_flag(status, QDG_FLAG_BAD_ZERO_POINT);
      const uint32_t nego = 0xC300u | (zq & 0x7Fu);  // bf16 of -(128 + zq)
      u32x2_t rec = {__builtin_bit_cast(uint32_t, s), nego | (nego << 16)};
      *((u32x2_t*)sdst + unit * 16 + col) = rec;
    }
  } else if (fmt == FMT_W4A16 || fmt == FMT_W4A8) {
    const uint32_t* src = (const uint32_t*)(qw + (e * N + (valid ? n : 0)) * (K / 2));
    u32x4_t out;
    for (int d = 0; d < 4; ++d) {
      uint32_t v;
      if (fmt == FMT_W4A16) {
        // dword d = K step j=d: elements 2i <- k+i, 2i+1 <- k+4+i, k = 128g+32c+8d
        const int64_t k0 = g * 128 + 32 * c + 8 * d;
        const int perm[8] = {0, 2, 4, 6, 1, 3, 5, 7};
        v = valid ? permute_nibbles(src[k0 / 8], perm) : 0u;
        if (wtype == QDG_W_INT4) v ^= 0x88888888u;  // two's complement -> biased q+8
      } else {
        // dword d = step j=d/2, half h=d%2; bytes of the unpacked int8 operand
        // come from even nibbles (low results) and odd nibbles (high results)
        const int64_t k0 = g * 128 + 32 * c + 16 * (d >> 1) + 8 * (d & 1);
        const int perm[8] = {0, 4, 1, 5, 2, 6, 3, 7};
        v = valid ? permute_nibbles(src[k0 / 8], perm) : 0u;
      }
      out[d] = v;
    }
    *((u32x4_t*)(wdst + unit * kUnit4Bytes) + lane) = out;
    if (c == 0) {
      const uint16_t* sc = (const uint16_t*)scales;
      const float s = valid ? half_bits_to_float(sc[(e * N + n) * groups + g]) : 0.f;
      if (!finite_f32(s)) raise_flag(status, QDG_FLAG_BAD_SCALE);
      if (fmt == FMT_W4A16) {
        uint32_t zq = 8;  // symmetric: q + 8 is stored, offset 128 + 8
        if (wtype == QDG_W_UINT4) zq = valid ? zeros[(e * N + n) * groups + g] : 0;
        if (zq > 15) raise_flag(status, QDG_FLAG_BAD_ZERO_POINT);
        const uint32_t nego = 0xC300u | (zq & 0x7Fu);  // bf16 of -(128 + zq)
        u32x2_t rec = {__builtin_bit_cast(uint32_t, s), nego | (nego << 16)};
        *((u32x2_t*)sdst + unit * 16 + col) = rec;
      } else {
        // the unpacked int8 operand is 16*q; fold 1/16 into the scale (exact)
        ((float*)sdst)[unit * 16 + col] = s * 0.0625f;
      }
    }
  } else if (fmt == FMT_MXFP4 || fmt == FMT_W4A4 || fmt == FMT_MXFP4_I8) {  // one weight layout for every activation type
    u32x4_t out = {0, 0, 0, 0};
    if (valid) out = *(const u32x4_t*)(qw + (e * N + n) * (K / 2) + (g * 128 + 32 * c) / 2);
    *((u32x4_t*)(wdst + unit * kUnit4Bytes) + lane) = out;
    uint8_t sc = 127;
    if (valid) {
      sc = ((const uint8_t*)scales)[(e * N + n) * (K / 32) + 4 * g + c];
      if (sc == 255) {
        sc = 254;
        raise_flag(status, QDG_FLAG_BAD_SCALE);
      }
    }
    sdst[unit * 64 + lane] = sc;
  } else if (fmt == FMT_NVFP4) {
    // codes as for MXFP4; the record of a lane holds the E4M3 codes of its
    // two 16-blocks (8g + 2c, 8g + 2c + 1); the NaN codes become +-448. The
    // expert's tensor scale leads its scale region.
    u32x4_t out = {0, 0, 0, 0};
    if (valid) out = *(const u32x4_t*)(qw + (e * N + n) * (K / 2) + (g * 128 + 32 * c) / 2);
    *((u32x4_t*)(wdst + unit * kUnit4Bytes) + lane) = out;
    uint32_t rec = 0;
    if (valid) {
      const uint8_t* sc = (const uint8_t*)scales + (e * N + n) * (K / 16) + 8 * g + 2 * c;
      uint32_t s0 = sc[0], s1 = sc[1];
      if ((s0 & 0x7Fu) == 0x7Fu || (s1 & 0x7Fu) == 0x7Fu) raise_flag(status, QDG_FLAG_BAD_SCALE);
      if ((s0 & 0x7Fu) == 0x7Fu) s0 -= 1;
      if ((s1 & 0x7Fu) == 0x7Fu) s1 -= 1;
      rec = s0 | (s1 << 8);
    }
    ((uint16_t*)(sdst + 256))[unit * 64 + lane] = (uint16_t)rec;
    if (unit == 0 && lane == 0) {
      const float ts = tscale[e];
      if (!finite_f32(ts)) raise_flag(status, QDG_FLAG_BAD_SCALE);
      *(float*)sdst = ts;
    }
  } else {  // FMT_W8A8: unit = [step j][lane][16 bytes]
    for (int j = 0; j < 2; ++j) {
      u32x4_t out = {0, 0, 0, 0};
      if (valid) out = *(const u32x4_t*)(qw + (e * N + n) * K + g * 128 + 32 * c + 16 * j);
      *((u32x4_t*)(wdst + unit * kUnit8Bytes) + j * 64 + lane) = out;
    }
    if (c == 0 && g == 0) {
      const float s = valid ? ((const float*)scales)[e * N + n] : 0.f;
      if (!finite_f32(s)) raise_flag(status, QDG_FLAG_BAD_SCALE);
      ((float*)sdst)[tile * 16 + col] = s;
    }
  }
}

// ------------------------------------------------------------ quantizers
// binary32 decisions with correctly rounded division and RNE, so the codes
// match any other implementation that follows the same binary32 steps.

__device__ __forceinline__ float f16_round(float x) { return (float)(_Float16)x; }

__device__ __forceinline__ uint32_t e2m1_rne_sat(float v) {
  const float a = fabsf(v);
  uint32_t code;
  if (a <= 0.25f) code = 0;
  else if (a < 0.75f) code = 1;
  else if (a <= 1.25f) code = 2;
  else if (a < 1.75f) code = 3;
  else if (a <= 2.5f) code = 4;
  else if (a < 3.5f) code = 5;
  else if (a <= 5.0f) code = 6;
  else code = 7;
  return code | (__builtin_signbit(v) ? 8u : 0u);
}

// One thread per quantization group (or per row for int8 per-channel).
__global__ void quantize_weights_kernel(int wtype, const float* __restrict__ w, uint8_t* __restrict__ qw,
                                        void* __restrict__ scales, uint8_t* __restrict__ zeros,
                                        int64_t rows, int64_t K, int group) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t gpr = K / group;  // groups per row
  if (tid >= rows * gpr) return;
  const int64_t row = tid / gpr, g = tid % gpr;
  const float* src = w + row * K + g * group;
  if (wtype == QDG_W_INT4 || wtype == QDG_W_UINT4 || wtype == QDG_W_UINT2) {
    float mn = src[0], mx = src[0], amax = 0.f;
    for (int i = 0; i < group; ++i) {
      const float v = src[i];
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
      amax = fmaxf(amax, fabsf(v));
    }
    uint8_t* dst = qw + row * (K / 2) + g * group / 2;
    _Float16* sc = (_Float16*)scales + row * gpr + g;
    if (wtype == QDG_W_UINT2) {  // the asymmetric rule with 2-bit codes, four per byte
      float s = f16_round(__fdiv_rn(mx - mn, 3.0f));
      if (s == 0.f) s = 1.0f;
      *sc = (_Float16)s;
      const float z = fminf(fmaxf(rintf(__fdiv_rn(-mn, s)), 0.f), 3.f);
      zeros[row * gpr + g] = (uint8_t)z;
      uint8_t* dst2 = qw + row * (K / 4) + g * group / 4;
      for (int i = 0; i < group; i += 4) {
        uint32_t b = 0;
        for (int j = 0; j < 4; ++j)
          b |= (uint32_t)fminf(fmaxf(rintf(__fdiv_rn(src[i + j], s)) + z, 0.f), 3.f) << (2 * j);
        dst2[i / 4] = (uint8_t)b;
      }
    } else if (wtype == QDG_W_INT4) {
      float s = f16_round(__fdiv_rn(amax, 7.0f));
      if (s == 0.f) s = 1.0f;
      *sc = (_Float16)s;
      for (int i = 0; i < group; i += 2) {
        const int q0 = (int)fminf(fmaxf(rintf(__fdiv_rn(src[i], s)), -8.f), 7.f);
        const int q1 = (int)fminf(fmaxf(rintf(__fdiv_rn(src[i + 1], s)), -8.f), 7.f);
        dst[i / 2] = (uint8_t)((q0 & 0xF) | ((q1 & 0xF) << 4));
      }
    } else {
      float s = f16_round(__fdiv_rn(mx - mn, 15.0f));
      if (s == 0.f) s = 1.0f;
      *sc = (_Float16)s;
      const float z = fminf(fmaxf(rintf(__fdiv_rn(-mn, s)), 0.f), 15.f);
      zeros[row * gpr + g] = (uint8_t)z;
      for (int i = 0; i < group; i += 2) {
        const int q0 = (int)fminf(fmaxf(rintf(__fdiv_rn(src[i], s)) + z, 0.f), 15.f);
        const int q1 = (int)fminf(fmaxf(rintf(__fdiv_rn(src[i + 1], s)) + z, 0.f), 15.f);
        dst[i / 2] = (uint8_t)(q0 | (q1 << 4));
      }
    }
  } else if (wtype == QDG_W_INT8) {
    float amax = 0.f;
    for (int64_t i = 0; i < K; ++i) amax = fmaxf(amax, fabsf(src[i]));
    float s = __fdiv_rn(amax, 127.0f);
    if (s == 0.f) s = 1.0f;
    ((float*)scales)[row] = s;
    int8_t* dst = (int8_t*)qw + row * K;
    for (int64_t i = 0; i < K; ++i)
      dst[i] = (int8_t)fminf(fmaxf(rintf(__fdiv_rn(src[i], s)), -127.f), 127.f);
  } else {  // MXFP4, group = 32
    float amax = 0.f;
    for (int i = 0; i < group; ++i) amax = fmaxf(amax, fabsf(src[i]));
    uint8_t* dst = qw + row * (K / 2) + g * group / 2;
    uint8_t* sc = (uint8_t*)scales + row * gpr + g;
    if (amax == 0.f) {
      *sc = 0;
      for (int i = 0; i < group / 2; ++i) dst[i] = 0;
      return;
    }
    const uint32_t u = __builtin_bit_cast(uint32_t, amax);
    const int ef = (int)((u >> 23) & 0xFF);
    int fl;  // floor(log2(amax))
    if (ef == 0) fl = (31 - __builtin_clz(u & 0x7FFFFFu)) - 149;
    else fl = ef - 127;
    const int x = min(max(fl - 2, -127), 127);
    *sc = (uint8_t)(x + 127);
    for (int i = 0; i < group; i += 2) {
      const uint32_t c0 = e2m1_rne_sat(ldexpf(src[i], -x));
      const uint32_t c1 = e2m1_rne_sat(ldexpf(src[i + 1], -x));
      dst[i / 2] = (uint8_t)(c0 | (c1 << 4));
    }
  }
}

// ------------------------------------------------------------ NVFP4 producer
// The per-expert tensor scale needs the whole tensor: zero the per-expert
// amax slots, take the amax with one atomic max per wave (non-negative
// binary32 values order like their bit patterns), turn it into the tensor
// scale, then quantize one 16-block per thread with the binary32 steps
// ts = f32(amax / 2688) (1 for an all-zero tensor),
// sb = e4m3_rne(min(f32(f32(amax_b / 6) / ts), 448)),
// q = e2m1_rne_sat(f32(w / f32(e4m3(sb) * ts))) (all zero when that is 0).
__global__ void nvfp4_zero_kernel(uint32_t* __restrict__ slots, int64_t experts) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < experts) slots[i] = 0u;
}
__global__ void nvfp4_amax_kernel(const float* __restrict__ w, int64_t per_expert, uint32_t* __restrict__ slots) {
  const int64_t e = blockIdx.y;
  const float* src = w + e * per_expert;
  float m = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < per_expert; i += (int64_t)gridDim.x * blockDim.x)
    m = fmaxf(m, fabsf(src[i]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) atomicMax(slots + e, __builtin_bit_cast(uint32_t, m));
}
__global__ void nvfp4_scale_kernel(uint32_t* __restrict__ slots, int64_t experts) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= experts) return;
  const float amax = __builtin_bit_cast(float, slots[e]);
  float ts = amax > 0.f ? __fdiv_rn(amax, 2688.0f) : 1.0f;
  if (ts == 0.f) ts = 1.0f;
  slots[e] = __builtin_bit_cast(uint32_t, ts);  // now the tensor scale
}
__global__ void nvfp4_quantize_kernel(const float* __restrict__ w, uint8_t* __restrict__ qw, uint8_t* __restrict__ sc,
                                      const float* __restrict__ ts_e, int64_t rows_per_expert, int64_t K,
                                      int64_t blocks) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= blocks) return;
  const int64_t bpr = K / 16;
  const int64_t row = tid / bpr, b = tid % bpr;
  const float ts = ts_e[row / rows_per_expert];
  const float* src = w + row * K + b * 16;
  float amax = 0.f;
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(src[i]));
  const float r = __fdiv_rn(__fdiv_rn(amax, 6.0f), ts);
  const uint32_t code = e4m3_rne(fminf(r, 448.0f));
  sc[tid] = (uint8_t)code;
  const float den = __fmul_rn(e4m3_to_f32(code), ts);
  uint8_t* dst = qw + row * (K / 2) + b * 8;
  for (int i = 0; i < 16; i += 2) {
    uint32_t c0 = 0, c1 = 0;
    if (den > 0.f) {
      c0 = e2m1_rne_sat(__fdiv_rn(src[i], den));
      c1 = e2m1_rne_sat(__fdiv_rn(src[i + 1], den));
    }
    dst[i / 2] = (uint8_t)(c0 | (c1 << 4));
  }
}

}  // namespace

hipError_t launch_preprocess(const qdg_layer_config& L, Format f, const PackedGeom& g,
                             const qdg_std_weights& w, void* packed, uint32_t* status, hipStream_t s) {
  const int64_t threads = g.experts * g.ntiles * g.groups * 64;
  const int bs = 256;
  const int64_t blocks = (threads + bs - 1) / bs;
  hipLaunchKernelGGL(repack_kernel, dim3((unsigned)blocks), dim3(bs), 0, s, (int)f, (int)L.wtype,
                     (const uint8_t*)w.qweight, w.scales, (const uint8_t*)w.zeros, (const float*)w.tensor_scale,
                     (uint8_t*)packed, g.n,
                     g.k, g.ntiles, g.groups, g.expert_stride, g.s_offset, g.experts, status);
  return hipGetLastError();
}

hipError_t launch_quantize_weights(const qdg_layer_config& L, const float* w, void* qweight,
                                   void* scales, void* zeros, hipStream_t s) {
  const int64_t rows = L.n * L.num_experts;
  if (L.wtype == QDG_W_NVFP4) {  // `zeros` receives the f32 tensor scale of each expert
    uint32_t* slots = (uint32_t*)zeros;
    const int64_t E = L.num_experts, per_expert = L.n * L.k;
    hipLaunchKernelGGL(nvfp4_zero_kernel, dim3((unsigned)((E + 255) / 256)), dim3(256), 0, s, slots, E);
    const int64_t bx = (per_expert + 256 * 16 - 1) / (256 * 16);
    hipLaunchKernelGGL(nvfp4_amax_kernel, dim3((unsigned)(bx < 1024 ? bx : 1024), (unsigned)E), dim3(256), 0, s, w,
                       per_expert, slots);
    hipLaunchKernelGGL(nvfp4_scale_kernel, dim3((unsigned)((E + 255) / 256)), dim3(256), 0, s, slots, E);
    const int64_t blocks = rows * (L.k / 16);
    hipLaunchKernelGGL(nvfp4_quantize_kernel, dim3((unsigned)((blocks + 255) / 256)), dim3(256), 0, s, w,
                       (uint8_t*)qweight, (uint8_t*)scales, (const float*)zeros, (int64_t)L.n, (int64_t)L.k, blocks);
    return hipGetLastError();
  }
  int group = L.wtype == QDG_W_INT8 ? (int)L.k : L.wtype == QDG_W_MXFP4 ? 32 : L.group_size;
  const int64_t threads = rows * (L.k / group);
  const int bs = 256;
  hipLaunchKernelGGL(quantize_weights_kernel, dim3((unsigned)((threads + bs - 1) / bs)), dim3(bs), 0, s,
                     (int)L.wtype, w, (uint8_t*)qweight, scales, (uint8_t*)zeros, rows, (int64_t)L.k, group);
  return hipGetLastError();
}

}  // namespace qdg
