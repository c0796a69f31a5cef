// Internal (not exported) interface between the C-ABI layer and the kernels.
#pragma once
#ifndef __HIPCC_RTC__
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>
#endif

#include "qdg.h"

namespace qdg {

enum Format {
  FMT_W4A16 = 0,
  FMT_W8A8 = 1,
  FMT_W4A8 = 2,
  FMT_MXFP4 = 3,
  FMT_W4A4 = 4,
  FMT_W8A16 = 5,
  FMT_NVFP4 = 6,
  FMT_MXFP4_I8 = 7,  // MXFP4 weights, per-token int8 activations
  FMT_W2A16 = 8      // uint2 weights (zero points), bf16 activations
};

// Geometry of the packed buffer of one layer.
struct PackedGeom {
  int64_t n, k, n_pad, ntiles, groups;
  int64_t w_bytes;        // weight units of one expert
  int64_t s_offset;       // offset of the scale records inside an expert
  int64_t s_bytes;        // scale records of one expert
  int64_t expert_stride;  // bytes per expert (256-aligned)
  int64_t experts;
};

PackedGeom packed_geom(const qdg_layer_config& L, Format f);

// Sets the thread's last-error message and returns st (for C-ABI entry
// points defined outside api.cpp).
qdg_status report_error(qdg_status st, const char* msg);
Format format_of(const qdg_layer_config& L);

// Kernel arguments shared by all GEMM kernels (passed by value).
struct GemmArgs {
  const void* A;
  const float* a_scales;
  const uint8_t* packed;
  void* Y;
  int M, N, K, groups, ntiles;
  int64_t expert_stride, s_offset;
  int otype;
  int split;            // K partitions reduced through the workspace
  void* partial;        // fp32 / int32 split partials
  unsigned* counters;   // reserved (the first 64 KiB of the workspace)
  // grouped MoE
  const int* sorted_ids;
  const int* block_expert;
  const int* num_padded;
  int top_k, a_per_pair, num_pairs;
  int epi;              // output epilogue (QDG_EPI_*)
  // large-M W4A16: per (group, row) negated row sums of A
  const float* rowsum;
  int m_pad;
  // unpack constants, passed at run time so the compiler keeps them in
  // registers (0x000F000F and 0x43004300)
  uint32_t unpack_mask, unpack_exp;
  // bytes of A (the streaming family reads A through a buffer resource of
  // this size: < 2^31, checked by the host)
  int64_t a_bytes;
};

// A kernel instance of the streaming (small-M) family.
struct StreamCfg {
  int mt;     // 16-row M tiles per workgroup (1, 2, 4)
  int nt;     // 16-column N tiles per workgroup
  int kw;     // wavefronts per workgroup (split the K range inside the WG)
  int split;  // K partitions across workgroups
};

// A kernel instance of the LDS-tiled (large-M) family.
struct TileCfg {
  int bm, bn, waves;
};

#ifndef __HIPCC_RTC__  // host launchers (not part of a run-time compiled kernel)
// The source files whose kernels can be compiled at run time (their text is
// embedded in the library), and one launch of such a kernel: its name
// expression in that source, grid and block, and its arguments (the
// GemmArgs, plus the row- and column-block counts for the LDS-tiled kernels).
enum JitSource { JIT_SRC_STREAM, JIT_SRC_TILE, JIT_SRC_WSTREAM, JIT_SRC_QTILE, JIT_SRC_WSTREAM8, JIT_NSRC };
struct KernelLaunch {
  int src;
  char expr[192];
  unsigned grid[3], block;
  bool mn_args;
  int m_blocks, n_blocks;
};

// The main-kernel launchers of the families. With desc set, they describe
// the launch they would make (kernel and grid) instead of making it, and
// launch nothing else (weight streaming then leaves the split reduce to
// the caller).
hipError_t launch_stream(Format f, bool asym, bool moe, const StreamCfg& c, const GemmArgs& a,
                         int grid_m_blocks, hipStream_t s);
hipError_t launch_tile(Format f, bool asym, bool moe, const TileCfg& c, const GemmArgs& a,
                       int grid_m_blocks, hipStream_t s, KernelLaunch* desc = nullptr);
hipError_t launch_reduce_splits(const GemmArgs& a, int m_pad, int n_pad, hipStream_t s);
hipError_t launch_wstream(bool asym, bool moe, const GemmArgs& a, int nsplit, int grid_m, hipStream_t s,
                          KernelLaunch* desc = nullptr);
// pad_skip (grouped MoE): the instance that skips the all-padding 32-row
// halves of expert blocks
hipError_t launch_qtile(Format f, bool moe, int bm, bool pad_skip, const GemmArgs& a, int m_blocks, hipStream_t s,
                        KernelLaunch* desc = nullptr);
hipError_t launch_wstream8(Format f, const GemmArgs& a, int nsplit, int nt, hipStream_t s,
                           KernelLaunch* desc = nullptr);
int wstream8_max_groups();
bool stream_cfg_supported(Format f, const StreamCfg& c);
bool tile_cfg_supported(Format f, const TileCfg& c);

hipError_t launch_rowsum(const void* a_bf16, const int* sorted_ids, const int* num_padded,
                         int top_k, int a_per_pair, int num_pairs, int M, int K, int m_pad,
                         float factor, float* out, hipStream_t s);

hipError_t launch_preprocess(const qdg_layer_config& L, Format f, const PackedGeom& g,
                             const qdg_std_weights& w, void* packed, uint32_t* status, hipStream_t s);
hipError_t launch_quantize_weights(const qdg_layer_config& L, const float* w, void* qweight,
                                   void* scales, void* zeros, hipStream_t s);
hipError_t launch_quantize_act(int atype, const void* a, int64_t M, int64_t K, void* qa,
                               float* scales, hipStream_t s);
// int8 activation codes [rows][K] -> E4M3 planes [rows][2K]: per 128-wide
// group g, bytes 256g .. 256g+127 hold hi = q >> 4 and 256g+128 .. 256g+255
// hold lo = q & 15 of the group's K values (q = 16 hi + lo, both exact).
hipError_t launch_act_i8_planes(const int8_t* qa, int64_t rows, int64_t K, uint8_t* planes, hipStream_t s);
hipError_t launch_moe_combine(const void* y, bool y_bf16, const float* w, int64_t T, int top_k, int64_t n,
                              void* out, int otype, hipStream_t s);
// Run-time compiled streaming-family instance (hipRTC): the loaded kernel,
// or an error. from_cache: 0 compiled now, 1 code object read from the cache
// directory, 2 already loaded in this process.
struct JitResult {
  hipFunction_t fn;
  double compile_ms, load_ms;
  int from_cache, code_bytes;
  char key[32];
  std::string lowered, error;
};
JitResult jit_stream_kernel(Format f, bool asym, bool raw, const StreamCfg& c, bool moe, const char* cache_dir);
hipError_t launch_stream_jit(hipFunction_t fn, const StreamCfg& c, const GemmArgs& a, int grid_m, hipStream_t s);
// The kernel a KernelLaunch names, compiled from its embedded source (same
// cache and load rules as jit_stream_kernel), and its launch.
JitResult jit_kernel(int src, const char* expr, const char* cache_dir);
hipError_t launch_jit(hipFunction_t fn, const KernelLaunch& d, const GemmArgs& a, hipStream_t s);

hipError_t launch_moe_align(const int32_t* topk_ids, int64_t T, int top_k, int E, int block_m,
                            int64_t capacity, int32_t* sorted_ids, int32_t* block_expert,
                            int32_t* num_padded, uint32_t* status, hipStream_t s);

#endif

}  // namespace qdg
