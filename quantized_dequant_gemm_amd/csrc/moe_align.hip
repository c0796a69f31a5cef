// Expert sort for the grouped MoE GEMM: (token, slot) pairs ordered by
// expert, ascending flat index within an expert, each expert padded to a
// multiple of block_m. One workgroup of 16 wavefronts:
//   1. each wave counts experts over its contiguous slice of the pair list
//      (LDS atomics; order does not matter for counts);
//   2. per expert: total, padded size, exclusive scan -> segment offsets, and
//      the start of each wave's run inside the segment;
//   3. each wave walks its slice 64 pairs at a time; lanes with the same
//      expert are found with one ballot per expert-id bit, the rank among
//      them is a popcount, so every pair lands at a unique, order-preserving
//      position without any atomics (the result is deterministic).
// The pages motivate MoE (each token activates a few experts while all are
// stored; kinachrichten, "Warum quantisierte Kernel wichtig sind") and name
// the grouped MoE path (jetabc, "跑得有多快"); the sort itself is a reading.
#include "qdg_device.h"
#include "qdg_internal.h"

namespace qdg {
namespace {

constexpr int kWaves = 16;
constexpr int kMaxE = 1024;
constexpr int kU = 8;  // 64-pair chunks whose loads are issued together

__global__ __launch_bounds__(1024) void moe_align_kernel(const int32_t* __restrict__ ids, int total, int E,
                                                         int bm, int capacity, int32_t* __restrict__ sorted_ids,
                                                         int32_t* __restrict__ block_expert,
                                                         int32_t* __restrict__ num_padded,
                                                         uint32_t* __restrict__ status) {
  __shared__ int cnt[kWaves][kMaxE];
  __shared__ int off[kMaxE + 1];
  __shared__ int scan_tmp[1024];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kWaves * kMaxE; i += 1024) (&cnt[0][0])[i] = 0;
  __syncthreads();
  const int slice = (total + kWaves - 1) / kWaves;
  const int lo = min(total, wave * slice), hi = min(total, lo + slice);
  // kU loads of the slice go out before their counts, so that a long slice
  // costs one load latency per kU * 64 pairs, not one per 64
  for (int base = lo; base < hi; base += kU * 64) {
    int ev[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = base + u * 64 + lane;
      ev[u] = i < hi ? ids[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int e = ev[u];
      if (base + u * 64 + lane >= hi) continue;
      if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[wave][e], 1);
      else if (status) atomicOr(status, QDG_FLAG_BAD_EXPERT_ID);  // the pair is left out
    }
  }
  __syncthreads();

  // per-expert totals and padded sizes; block-wide exclusive scan (E <= 1024)
  int padded = 0, tot = 0;
  if (tid < E) {
    for (int w = 0; w < kWaves; ++w) tot += cnt[w][tid];
    padded = (tot + bm - 1) / bm * bm;
  }
  scan_tmp[tid] = padded;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int v = tid >= d ? scan_tmp[tid - d] : 0;
    __syncthreads();
    scan_tmp[tid] += v;
    __syncthreads();
  }
  const int excl = scan_tmp[tid] - padded;
  if (tid < E) {
    off[tid] = excl;
    // start of each wave's run inside the expert's segment
    int run = excl;
    for (int w = 0; w < kWaves; ++w) {
      const int c = cnt[w][tid];
      cnt[w][tid] = run;
      run += c;
    }
    // padding slots of this expert hold the sentinel
    for (int p = excl + tot; p < excl + padded; ++p) sorted_ids[p] = total;
    for (int b = excl / bm; b < (excl + padded) / bm; ++b) block_expert[b] = tid;
  }
  if (tid == 1023) off[kMaxE] = scan_tmp[1023];
  __syncthreads();
  const int npad = off[kMaxE];
  if (tid == 0) *num_padded = npad;
  for (int p = npad + tid; p < capacity; p += 1024) sorted_ids[p] = total;
  for (int b = npad / bm + tid; b < capacity / bm; b += 1024) block_expert[b] = -1;

  // stable scatter, one wave per slice, 64 pairs per step
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = lo; base < hi; base += kU * 64) {
    int ev[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = base + u * 64 + lane;
      ev[u] = i < hi ? ids[i] : -1;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      // chunks in order: the runs of chunk u start after those of u - 1
      const int i = base + u * 64 + lane;
      const int e = ev[u];
      const bool valid = (unsigned)e < (unsigned)E;
      uint64_t same = __ballot(valid);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = valid && ((e >> b) & 1);
        const uint64_t ones = __ballot(bit);
        same &= bit ? ones : ~ones;
      }
      if (valid) {
        const int rank = __popcll(same & lt);
        const int n = __popcll(same);
        const int pos = cnt[wave][e] + rank;
        sorted_ids[pos] = i;
        if (rank == n - 1) cnt[wave][e] += n;  // one writer per expert
      }
    }
  }
}

// Top-k weighted combine: one thread per (token, 4 columns). The top_k pair
// rows of a token are added in ascending slot order (deterministic).
// y rows in fp32 (YB16 = false) or bf16 (YB16 = true, widened exactly to
// fp32 before the multiply); the sum is the same fp32 FMA chain in ascending
// j either way.
template <bool YB16>
__global__ void moe_combine_kernel(const void* __restrict__ yv, const float* __restrict__ w, int64_t T,
                                   int top_k, int64_t n, void* __restrict__ out, int otype) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_row = n / 4;
  if (q >= T * per_row) return;
  const int64_t t = q / per_row, c = (q % per_row) * 4;
  float s[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < top_k; ++j) {
    const int64_t r = t * top_k + j;
    const float wj = w[r];
    float v[4];
    if constexpr (YB16) {
      const uint2 h = *(const uint2*)((const uint16_t*)yv + r * n + c);
      v[0] = __builtin_bit_cast(float, h.x << 16);
      v[1] = __builtin_bit_cast(float, h.x & 0xFFFF0000u);
      v[2] = __builtin_bit_cast(float, h.y << 16);
      v[3] = __builtin_bit_cast(float, h.y & 0xFFFF0000u);
    } else {
      const float4 f = *(const float4*)((const float*)yv + r * n + c);
      v[0] = f.x;
      v[1] = f.y;
      v[2] = f.z;
      v[3] = f.w;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] = __builtin_fmaf(wj, v[e], s[e]);
  }
  if (otype == QDG_O_F32) {
    *(float4*)((float*)out + t * n + c) = make_float4(s[0], s[1], s[2], s[3]);
  } else {
    uint16_t* o = (uint16_t*)out + t * n + c;
    for (int e = 0; e < 4; ++e) o[e] = (uint16_t)f32_to_bf16_rne(s[e]);
  }
}

}  // namespace

hipError_t launch_moe_combine(const void* y, bool y_bf16, const float* w, int64_t T, int top_k, int64_t n,
                              void* out, int otype, hipStream_t s) {
  const int64_t threads = T * (n / 4);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (y_bf16)
    hipLaunchKernelGGL(moe_combine_kernel<true>, grid, dim3(256), 0, s, y, w, T, top_k, n, out, otype);
  else
    hipLaunchKernelGGL(moe_combine_kernel<false>, grid, dim3(256), 0, s, y, w, T, top_k, n, out, otype);
  return hipGetLastError();
}

hipError_t launch_moe_align(const int32_t* topk_ids, int64_t T, int top_k, int E, int block_m,
                            int64_t capacity, int32_t* sorted_ids, int32_t* block_expert,
                            int32_t* num_padded, uint32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(moe_align_kernel, dim3(1), dim3(1024), 0, s, topk_ids, (int)(T * top_k), E, block_m,
                     (int)capacity, sorted_ids, block_expert, num_padded, status);
  return hipGetLastError();
}

}  // namespace qdg
