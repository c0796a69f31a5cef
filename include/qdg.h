/*
 * qdg.h -- C ABI of libqdg.so, a fused dequantize-and-multiply GEMM library for
 * AMD Instinct MI355X (gfx950 / CDNA4).
 *
 * It computes Y = A * dequant(Wq, scales, zeros)^T for a linear layer whose
 * weight W is stored [N, K] in a quantized "standard format", plus the
 * expert-grouped MoE form of the same product.
 *
 * Design taken from the pages on the Humming kernel library:
 *  - one standard representation of weights, scales and zero points, into
 *    which every export format is brought; a preprocessing step then checks
 *    the parameters, pads dimensions and repacks the tensors for the target
 *    kernel (kinachrichten, "Wie die Architektur funktioniert");
 *  - a kernel is described by a Layer config (shapes, types, quantization
 *    parameters, target architecture), a Compute config (GEMM kind and options
 *    such as batch invariance) and a Tuning config (tiles, pipeline, MMA
 *    instruction); device heuristics fill the Tuning config when none is given
 *    and different kernels may serve different input-size ranges (same
 *    section);
 *  - validation sits at the shared interface and unsupported combinations are
 *    rejected clearly, never served silently ("vLLM Humming: why shared
 *    quantization still needs specialized kernels", section "The architectural
 *    gain is a smaller maintenance surface"); the record of which
 *    implementation serves which combination is available
 *    (retrivium analysis, section "A compatibility example").
 *
 * Conventions for every entry point:
 *  - All tensor pointers are device pointers owned by the caller (hipMalloc or
 *    a framework allocator). The library keeps no tensor pointer after a call
 *    returns and never allocates device memory in a compute call.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Device work is enqueued asynchronously on it; host-side validation is
 *    synchronous and happens before anything is enqueued.
 *  - Every call returns a qdg_status. On anything but QDG_OK nothing has been
 *    enqueued (except QDG_ERR_HIP, reported when a launch fails) and
 *    qdg_last_error() returns a thread-local message.
 *  - Row-major layouts; "bf16" = IEEE binary32 upper half; "f16" = binary16.
 */
#ifndef QDG_H
#define QDG_H

#ifndef __HIPCC_RTC__
#include <stddef.h>
#include <stdint.h>
#endif

#ifdef __cplusplus
extern "C" {
#endif

#define QDG_LAYOUT_VERSION 1

typedef enum qdg_status {
  QDG_OK = 0,
  QDG_ERR_INVALID_ARG = 1, /* null pointer, negative or inconsistent size, bad enum */
  QDG_ERR_UNSUPPORTED = 2, /* a valid combination that no kernel instance serves */
  QDG_ERR_MISALIGNED = 3,  /* a pointer or row stride breaks the 16-byte rule */
  QDG_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required */
  QDG_ERR_HIP = 5          /* the HIP runtime reported an error */
} qdg_status;

/* Weight element types of the standard format. */
enum { QDG_W_INT4 = 0,  /* two's-complement 4-bit, symmetric (no zeros) */
       QDG_W_UINT4 = 1, /* unsigned 4-bit with uint8 zero points (asymmetric) */
       QDG_W_INT8 = 2,  /* int8, symmetric, one fp32 scale per output channel */
       QDG_W_MXFP4 = 3, /* OCP MX FP4 E2M1 with E8M0 scale per 32 along K */
       QDG_W_NVFP4 = 4, /* E2M1 with an E4M3 scale per 16 along K and one
                           binary32 scale per tensor (expert) */
       QDG_W_UINT2 = 5  /* unsigned 2-bit with uint8 zero points (asymmetric) */ };
/* Scale storage types. */
enum { QDG_S_F16 = 0, QDG_S_F32 = 1, QDG_S_E8M0 = 2, QDG_S_E4M3 = 3 };
/* Activation types. MXFP4 activations (W4A4): E2M1 codes u8 [M][k/2], two
   per byte with the even k in the low nibble, and E8M0 scale codes u8
   [M][k/32]; the qdg_gemm / qdg_moe_gemm a_scales pointer then carries the
   E8M0 bytes. */
enum { QDG_A_BF16 = 0, QDG_A_INT8 = 1, QDG_A_FP8E4M3 = 2, QDG_A_MXFP4 = 3 };
/* Output types. QDG_O_I32 returns the raw integer accumulator
   sum_k qa*qw (integer-weight paths only; every scale ignored). */
enum { QDG_O_BF16 = 0, QDG_O_F32 = 1, QDG_O_I32 = 2 };
/* GEMM kinds (Compute config). */
enum { QDG_KIND_DENSE = 0, QDG_KIND_MOE = 1 };

/* Layer config: what the layer is. The weight of one layer (one expert) is
   [n, k]. Supported combinations (anything else is QDG_ERR_UNSUPPORTED):
     W4A16      wtype INT4 (has_zeros 0) or UINT4 (has_zeros 1), stype F16,
                group_size 128, atype BF16, otype BF16 or F32
     W8A8       wtype INT8, stype F32 (per channel, group_size 0), atype INT8,
                act_group 0 (per token), otype BF16, F32 or I32
     W4A8-INT8  wtype INT4, stype F16, group_size 128, atype INT8, act_group 0,
                otype BF16, F32 or I32
     W4A8-MXFP4 wtype MXFP4, stype E8M0, group_size 32, atype FP8E4M3,
                act_group 128, otype BF16 or F32
     W4A8-MXFP4-INT8 wtype MXFP4, stype E8M0, group_size 32, atype INT8,
                act_group 0 (per token), otype BF16 or F32 (the pages' MXFP4 ->
                INT8 path: kinachrichten, "Das Wichtigste in Kürze"; each int8
                activation q is split exactly into 16 hi + lo, both E4M3, and
                the fp4 weights meet both planes in the scaled fp8 x fp4 MFMA,
                E8M0 applied by the hardware; streaming family at every M;
                the planes take 2 * rows * k bytes of the workspace)
     W4A4-MXFP4 wtype MXFP4, stype E8M0, group_size 32, atype MXFP4,
                act_group 32, otype BF16 or F32 (the pages list W4A4 among
                the common configurations: kinachrichten, "Warum
                quantisierte Kernel wichtig sind"; served by the streaming
                family with fp4 x fp4 scaled MFMAs, both E8M0 scales applied
                by the hardware)
     W4A16-NVFP4 wtype NVFP4, stype E4M3, group_size 16, atype BF16,
                act_group 0, otype BF16 or F32 (the pages name NVFP4 beside
                INT4 as a 4-bit format with its own number format and
                scaling: kinachrichten, "Warum quantisierte Kernel wichtig
                sind"; served by the streaming family: each E2M1 value times
                its E4M3 block scale is exact in bf16, so the weights enter
                the bf16 MFMA already scaled and the tensor scale is applied
                to the fp32 result)
     W2A16      wtype UINT2 (has_zeros 1), stype F16, group_size 128, atype
                BF16, act_group 0, otype BF16 or F32 (a WNA16 width: the pages
                list WNA16 without fixing N, kinachrichten, "Warum
                quantisierte Kernel wichtig sind"; the 4-bit asymmetric rule
                with 2-bit codes, streaming family at every M)
   Shapes: k a positive multiple of 128; n >= 1 (padded internally to a
   multiple of 16); num_experts >= 1 (1 for a dense layer). arch = 950. */
typedef struct qdg_layer_config {
  int64_t n, k, num_experts;
  int32_t wtype, stype, group_size, has_zeros;
  int32_t atype, act_group, otype, arch;
} qdg_layer_config;

/* Compute config: which computation. kind DENSE or MOE (MoE: W4A16 with
   INT4 symmetric weights, W8A8, W4A8-INT8, W4A8-MXFP4, W4A4-MXFP4, W8A16,
   W4A16-NVFP4; 128-row MoE blocks: W4A16, and W8A16 / W4A16-NVFP4 without
   an epilogue). batch_invariant = 1 makes row m of Y bitwise independent of M and
   of the other rows (one fixed reduction order for every M). top_k: MoE
   slots per token. */
typedef struct qdg_compute_config {
  int32_t kind, batch_invariant, top_k;
  int32_t epilogue; /* QDG_EPI_*; QDG_EPI_NONE for plain Y */
} qdg_compute_config;

/* Output epilogues of a MoE plan (the MoE block around the grouped GEMM:
   jetabc, "跑得有多快", names the grouped MoE path the library serves).
   QDG_EPI_SILU_MUL: the layer is a fused gate+up projection with n = 2*I
   output rows, rows [0, I) the gate and [I, 2I) the up projection (I a
   multiple of 16); Y is [T*top_k][I] with Y[r][i] = silu(G[r][i]) * U[r][i],
   silu(x) = x / (1 + exp(-x)), computed in fp32 from the fp32 GEMM results
   before the output conversion. Not for int32 output. */
enum { QDG_EPI_NONE = 0, QDG_EPI_SILU_MUL = 1 };

/* Tuning config: how to run. Zero in any field means "heuristic". Three
   kernel families exist; block_m and waves select one:
     weight streaming  block_m 16, block_n 64, waves 8 (W4A16 only; the
                       default for M <= 16 and 16-row MoE blocks)
     streaming         block_m 16, 32 or 64, block_n 16, 32 or 64, waves 4
                       (every format; the default otherwise for M <= 64)
     LDS-tiled         block_m 128 (block_n 256) or 256 (block_n 128), waves
                       8 or 4 (dense W4A16; the default from M = 65), and
                       block_m 64 with block_n 512, waves 8 (dense W4A16; the
                       default for M = 33 to 64); block_n 512 with block_m
                       16 or 0, waves 8 (grouped MoE W4A16: 16 x 512 tiles
                       for 16-row expert blocks); block_m 128, block_n 256,
                       waves 8 for dense W8A16, W4A16-NVFP4 and W2A16 (the
                       default from M = 33); the 8-bit activation formats
                       have their own 128 x 256 tiles (the default from
                       M = 64, or above 128 for W4A4 and narrow W8A8 layers)
   split_k is the number of K partitions (dense only), reduced in a fixed
   order. batch_invariant plans use the streaming family for every M. Fields
   block_k, stages, mfma and load_path are recorded in the description but
   only one value each is implemented (128, 2, 16, 0). */
typedef struct qdg_tuning_config {
  int32_t block_m, block_n, block_k, split_k;
  int32_t stages, waves, mfma, load_path;
} qdg_tuning_config;

/* Standard-format weights (device pointers; all experts back to back):
     INT4 / UINT4 / MXFP4 qweight  u8 [E][n][k/2], element k of a row in byte
                                   k/2, even k in the low nibble
     UINT2 qweight                 u8 [E][n][k/4], element k in byte k/4 at
                                   bits 2 (k % 4) .. 2 (k % 4) + 1
     INT8 qweight                  i8 [E][n][k]
     F16 scales                    f16 [E][n][k/group_size]
     F32 scales (INT8)             f32 [E][n]
     E8M0 scales (MXFP4)           u8 [E][n][k/32], value 2^(e-127); 255 invalid
     E4M3 scales (NVFP4)           u8 [E][n][k/16], OCP E4M3 codes; the NaN
                                   codes 0x7F / 0xFF are invalid
     zeros (UINT4, UINT2)          u8 [E][n][k/group_size], values 0..15
                                   (UINT2: 0..3)
     tensor_scale (NVFP4 only)     f32 [E], one scale per expert
   Dequantized weight: w = (q - z) * s, z = 0 when symmetric; MXFP4:
   w = e2m1(q) * 2^(e-127); NVFP4: w = e2m1(q) * e4m3(s) * tensor_scale.
   Pointers a format does not use may be NULL. */
typedef struct qdg_std_weights {
  const void* qweight;
  const void* scales;
  const void* zeros;
  const void* tensor_scale;
} qdg_std_weights;

typedef struct qdg_plan qdg_plan;

/* Input flags: bits that qdg_preprocess and qdg_moe_align OR into an
   optional caller-owned device status word (uint32_t, 4-byte aligned) when
   they meet input the standard format does not allow. The call still
   completes and its outputs are defined (noted per flag); a caller that
   passes the word zeroes it beforehand and reads it after the stream has
   run. The library never clears it, so one word can collect the flags of
   several calls. Concentrating validation at the shared interface and
   rejecting visibly is the pages' contract ("vLLM Humming: why shared
   quantization still needs specialized kernels", section "The architectural
   gain is a smaller maintenance surface"). */
enum {
  QDG_FLAG_BAD_SCALE = 1u,       /* a reserved or non-finite scale: E8M0 code
                                    255, an E4M3 NaN code (0x7F, 0xFF), a
                                    non-finite f16 / f32 scale or NVFP4 tensor
                                    scale. Packed as the largest finite scale
                                    of its sign (E8M0 254, E4M3 +-448); a
                                    non-finite f16 / f32 scale is packed as it is */
  QDG_FLAG_BAD_ZERO_POINT = 2u,  /* a UINT4 zero point above 15 (UINT2:
                                    above 3); packed modulo 128 */
  QDG_FLAG_BAD_EXPERT_ID = 4u    /* a top-k id outside [0, E); the pair is
                                    left out of every expert block, so its
                                    output row is never written */
};

/* Library identity: "qdg <version> gfx950 layout <QDG_LAYOUT_VERSION>". */
const char* qdg_version(void);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* qdg_last_error(void);

/* Checks a layer config against the supported combinations (host only). */
qdg_status qdg_validate_layer(const qdg_layer_config* layer);

/* Bytes of the packed (kernel-layout) buffer qdg_preprocess writes for this
   layer, all experts included. */
qdg_status qdg_preprocess_query(const qdg_layer_config* layer, size_t* packed_bytes);

/* Preprocess (once per layer, not part of steady-state timing; the pages'
   step that checks parameters, pads dimensions and repacks the standard
   format for the target kernel: kinachrichten, "Wie die Architektur
   funktioniert"): validates the layer, pads n to a multiple of 16 and
   rewrites the standard-format weights into the gfx950 MFMA fragment layout
   of the target kernels. `packed` (>= qdg_preprocess_query bytes, 256-byte
   aligned) is written entirely; the standard-format buffers are only read.
   Scale and zero-point values are checked on the device while they are
   packed: `status` (may be NULL; device, 4-byte aligned, caller-owned and
   caller-zeroed) receives QDG_FLAG_BAD_SCALE / QDG_FLAG_BAD_ZERO_POINT for
   the values the standard format forbids (see the flags). */
qdg_status qdg_preprocess(const qdg_layer_config* layer, const qdg_std_weights* weights,
                          void* packed, size_t packed_bytes, uint32_t* status, void* stream);

/* Quantize float32 weights [E][n][k] (device) into the standard format of
   `layer` (a producer of the standard format). Decisions are taken in
   binary32 with RNE:
     INT4  s = f16(amax/7),  q = clamp(rne(w/s), -8, 7), per group of 128
     UINT4 s = f16((max-min)/15), z = clamp(rne(-min/s), 0, 15),
           q = clamp(rne(w/s) + z, 0, 15)
     INT8  s = f32(amax/127), q = clamp(rne(w/s), -127, 127), per row
     MXFP4 X = floor(log2(amax)) - 2 per 32, e = X + 127, q = e2m1_rne_sat(w/2^X)
   A scale that is zero is stored as 1.0 (all-zero group). `zeros` is used
   for UINT4 only, except for NVFP4, where it receives the f32 [E] tensor
   scales:
     NVFP4 ts = f32(amax_tensor/2688) (1 if all zero) per expert,
           s = e4m3_rne(min(f32(f32(amax/6)/ts), 448)) per 16,
           q = e2m1_rne_sat(f32(w/f32(e4m3(s)*ts))) (0 where that is 0). */
qdg_status qdg_quantize_weights(const qdg_layer_config* layer, const float* w,
                                void* qweight, void* scales, void* zeros, void* stream);

/* Activation quantization for the W8A8 / W4A8 / W4A4 paths (layer->atype
   INT8, FP8E4M3 or MXFP4): the pages' formats lower the precision of the
   activations as well as of the weights (kinachrichten, "Warum
   quantisierte Kernel wichtig sind"; the A in W8A8, W4A8, W4A4 counts the
   activation bits: jetabc, "量化是怎么回事"); the rules below are this
   library's reading (the pages fix none). a_bf16 [M][k] row-major ->
     INT8:    qa i8 [M][k], a_scales f32 [M];       per token
     FP8E4M3: qa u8 E4M3 [M][k], a_scales f32 [M][k/128]; per 128-group
   with amax the largest |x|, inv = f32(Q/amax) (Q = 127 or 448),
   code = rne(clamp(f32(x*inv), -Q, Q)), scale = f32(amax/Q); amax = 0 gives
   scale 1 and zero codes;
     MXFP4:   qa u8 [M][k/2] E2M1 codes (even k in the low nibble), a_scales
              (as bytes) u8 E8M0 [M][k/32]: per block of 32 the MXFP4 rule of
              qdg_quantize_weights (an all-zero block stores E8M0 code 0 and
              zero codes; a negative value that rounds to zero keeps its sign).
   Bit-exact by construction (binary32, RNE). All pointers are device
   pointers owned by the caller; a_bf16 and qa 16-byte aligned, a_scales
   4-byte aligned (else QDG_ERR_MISALIGNED); M >= 0 (0 enqueues nothing).
   QDG_ERR_INVALID_ARG for NULL pointers or M < 0, QDG_ERR_UNSUPPORTED for
   a layer with bf16 activations or M >= 2^31. */
qdg_status qdg_quantize_act(const qdg_layer_config* layer, const void* a_bf16, int64_t M,
                            void* qa, float* a_scales, void* stream);

/* Build an execution plan (host only, no device work). tuning may be NULL
   (device heuristics per M range). The plan is immutable and may be shared
   across threads and streams; destroy it with qdg_plan_destroy. */
qdg_status qdg_plan_create(const qdg_layer_config* layer, const qdg_compute_config* compute,
                           const qdg_tuning_config* tuning, qdg_plan** out);
void qdg_plan_destroy(qdg_plan* plan);

/* Workspace bytes qdg_gemm / qdg_moe_gemm need for M rows (M = T for MoE).
   The scratch the kernel instance that serves M uses (the instance differs
   by M range: kinachrichten, "Wie die Architektur funktioniert"): fp32
   split-K partials (added by a second kernel in split order), the row sums
   of A for the LDS-tiled bf16 family, and the two E4M3 planes of the int8
   activations of the MXFP4 x INT8 path. Its contents need no
   initialisation (the first 64 KiB are reserved). Calls that share one
   workspace must be ordered on one stream. QDG_ERR_INVALID_ARG for a NULL
   plan or bytes, or M < 0. */
qdg_status qdg_plan_workspace(const qdg_plan* plan, int64_t M, size_t* bytes);

/* Writes a one-line record of the kernel instance that serves M rows (family,
   tiles, split, waves, MFMA shape, packed layout version, arch) into buf.
   Returns the length of the full record (snprintf semantics), -1 on error. */
int qdg_plan_describe(const qdg_plan* plan, int64_t M, char* buf, size_t len);

/* The same record for a grouped MoE call of T tokens with block_m-row expert
   blocks (16, 32, 64 or 128): the family and tiles qdg_moe_gemm runs.
   Returns the record length, -1 on error (not a MoE plan, bad block_m). */
int qdg_moe_describe(const qdg_plan* plan, int64_t T, int32_t block_m, char* buf, size_t len);

/* Dense GEMM Y[M][n] = dequant(A)[M][k] * dequant(W)^T: the quantized
   linear layer, weights (and for the 8- and 4-bit activation formats the
   activations) at reduced precision (kinachrichten, "Warum quantisierte
   Kernel wichtig sind"), dequantization and scaling applied inside the one
   kernel that feeds the matrix cores (kinachrichten, "Kompilierzeiten und
   gerätespezifisches Tuning"), the kernel instance picked per M range
   (kinachrichten, "Wie die Architektur funktioniert").
   A (row stride k elements, 16-byte aligned):
      bf16 [M][k]   W4A16 (INT4, UINT4), W8A16, W4A16-NVFP4, W2A16;
      i8 [M][k]     W8A8, W4A8-INT8, W4A8-MXFP4-INT8;
      E4M3 [M][k]   W4A8-MXFP4;
      u8 [M][k/2]   W4A4 (E2M1 codes, even k in the low nibble).
   a_scales: NULL for the bf16 formats; f32 [M] for the int8 formats
      (ignored, may be NULL, with otype I32); f32 [M][k/128] for W4A8-MXFP4;
      u8 E8M0 [M][k/32] for W4A4 (passed through this pointer).
   packed: the qdg_preprocess output for this layer (256-byte aligned).
   Y: [M][n] of otype (bf16, f32, or i32 for W8A8 / W4A8-INT8 only: the
      exact integer accumulators), row stride n, aligned to its element.
   M >= 0 (M = 0 enqueues nothing). workspace >= qdg_plan_workspace bytes,
   256-byte aligned. All pointers are device pointers owned by the caller.
   Errors: QDG_ERR_INVALID_ARG (NULL plan or operand, a MoE plan, M < 0),
   QDG_ERR_MISALIGNED, QDG_ERR_WORKSPACE, QDG_ERR_UNSUPPORTED (A beyond the
   serving family's addressing: 2 GiB streaming, 4 GiB tiled), QDG_ERR_HIP
   (a launch failed). */
qdg_status qdg_gemm(const qdg_plan* plan, const void* A, const float* a_scales, const void* packed,
                    void* Y, int64_t M, void* workspace, size_t ws_bytes, void* stream);

/* qdg_gemm without a workspace argument, for callers that cannot allocate
   device memory: code under HIP graph capture, tight serving loops,
   harnesses that forbid allocation. The workspace is a fixed device array
   of QDG_NOALLOC_SCRATCH_BYTES per GPU inside the library, held until the
   process ends; a call whose qdg_plan_workspace(plan, M) exceeds it returns
   QDG_ERR_WORKSPACE (use qdg_gemm with a caller workspace then). Every call
   on one GPU shares that GPU's array, so calls that overlap on one GPU
   (other streams or threads at the same time) race: order them on one
   stream. No call allocates or frees device memory. The first call on a
   device looks up that device's array address (host only, no allocation).
   Other arguments, results and errors as for qdg_gemm. */
#define QDG_NOALLOC_SCRATCH_BYTES (64ull << 20)
qdg_status qdg_gemm_noalloc(const qdg_plan* plan, const void* A, const float* a_scales, const void* packed,
                            void* Y, int64_t M, void* stream);

/* Run-time compilation (the pages build each kernel instance at run time
   from its configuration: kinachrichten, "Kompilierzeiten und
   gerätespezifisches Tuning"; jetabc, "Humming 的做法", item 3). Compiles
   with hipRTC the main kernel of the instance that serves M rows of the plan
   (for a MoE plan: T = M tokens in block_m-row blocks; block_m is ignored
   for dense plans), whichever family it belongs to (streaming, weight
   streaming, LDS-tiled, 8-bit LDS-tiled, 8-bit weight streaming), from that
   family's kernel source embedded in the library, loads it on the current
   device, and makes the plan launch it for every call that selects that
   instance ("code=jit" in the descriptions); the small helper kernels of a
   call (row sums, split reduce, activation planes) stay ahead of time. With
   a cache_dir (may be NULL) the code object is stored there, under a key of
   the kernel, the target, the options, the compiler version and the source
   text, and later processes load it instead of compiling. QDG_ERR_UNSUPPORTED
   when no instance serves M, and for W4A8-MXFP4 and W4A8-MXFP4-INT8 plans
   (their fp8 x fp4 scaled-MFMA instances gave results scaled by 2^-127 when
   launched from a hipRTC code object on MI355X; they run ahead of time); a
   compile or load failure QDG_ERR_HIP (with the compiler log in
   qdg_last_error). Blocks while compiling. The plan is
   modified: no other call may use it concurrently. */
typedef struct qdg_jit_info {
  double compile_ms;  /* hipRTC compile time; 0 when no compile was needed */
  double load_ms;     /* code object load time */
  int32_t from_cache; /* 0 compiled now, 1 read from cache_dir, 2 already loaded */
  int32_t code_bytes;
  char key[32];       /* cache key (hex) */
} qdg_jit_info;
qdg_status qdg_plan_jit(qdg_plan* plan, int64_t M, int32_t block_m, const char* cache_dir, qdg_jit_info* info);

/* Per-M-range autotuning of a dense plan (the pages' per-device tuning of
   the kernel instances per M range, with heuristics as the fallback:
   kinachrichten, "Kompilierzeiten und gerätespezifisches Tuning"; jetabc,
   "Humming 的做法", item 2). Times every kernel instance that can serve M
   rows (the heuristics' own instance, weight streaming with several K
   splits, streaming with every row block and tile count, LDS-tiled shapes)
   in three interleaved rounds of one untimed launch and reps launches
   between two events on stream. The timed launches rotate over copies of
   packed that together hold at least 512 MiB (twice the MI355X last-level
   cache), so no launch finds its weights cache-resident from the one
   before; the call allocates them with hipMalloc, frees them before it
   returns, and times on packed alone when the allocation fails. The
   instance with the lowest round time is recorded for M's range (M in
   (2^(b-1), 2^b], b = 0..31), except that the heuristics' instance is kept
   unless the winner is more than 3 % faster. Later
   qdg_gemm, qdg_plan_workspace and qdg_plan_describe calls with an M in that
   range use it ("tuning=autotuned"). Arguments as for qdg_gemm; instances
   whose workspace exceeds ws_bytes are skipped (query qdg_plan_workspace
   again afterwards). Blocks until the timing is done; Y holds the GEMM
   result of the chosen instance on return. chosen (may be NULL) receives
   the winning tuning, which a later plan may take as its user tuning;
   best_us (may be NULL) its time per launch in microseconds. Only dense
   plans without a user tuning and without batch invariance are tuned
   (else QDG_ERR_UNSUPPORTED); reps in [1, 1000]. The call modifies the
   plan: no other call may use the plan concurrently. */
qdg_status qdg_plan_autotune(qdg_plan* plan, const void* A, const float* a_scales, const void* packed, void* Y,
                             int64_t M, void* workspace, size_t ws_bytes, int32_t reps, void* stream,
                             qdg_tuning_config* chosen, float* best_us);

/* Forgets every autotuned range of the plan (the heuristics serve again).
   Not concurrently with other calls on the plan. */
qdg_status qdg_plan_autotune_reset(qdg_plan* plan);

/* Capacity (entries of sorted_ids) that qdg_moe_align may need:
   round_up(T*top_k + E*(block_m-1), block_m); block_expert needs
   capacity/block_m entries. */
qdg_status qdg_moe_align_capacity(int64_t T, int32_t top_k, int32_t num_experts, int32_t block_m,
                                  int64_t* capacity);

/* Expert sort for the grouped GEMM (the pages' grouped MoE path, jetabc,
   "跑得有多快", over tokens that each activate a few of the stored experts,
   kinachrichten, "Warum quantisierte Kernel wichtig sind"; the sort order
   is this library's reading). topk_ids i32 [T][top_k] (values in [0, E))
   -> pairs (flat index t*top_k+j) sorted by expert, ascending flat index
   within an expert, each expert padded to a multiple of block_m with the
   sentinel T*top_k; experts with no pair get no block.
   Outputs (capacity from qdg_moe_align_capacity): sorted_ids i32 [capacity]
   (entries past num_padded hold the sentinel), block_expert i32
   [capacity/block_m] (-1 past the last block), num_padded i32 [1].
   block_m in {16, 32, 64, 128}; 1 <= E <= 1024; 1 <= top_k <= 32;
   T*top_k <= 2^20. An id outside [0, E) is left out (its pair row of a
   later qdg_moe_gemm is not written) and sets QDG_FLAG_BAD_EXPERT_ID in
   `status` (may be NULL; device, caller-owned and caller-zeroed). */
qdg_status qdg_moe_align(const int32_t* topk_ids, int64_t T, int32_t top_k, int32_t num_experts,
                         int32_t block_m, int32_t* sorted_ids, int32_t* block_expert,
                         int32_t* num_padded, uint32_t* status, void* stream);

/* Grouped MoE GEMM (the pages' grouped MoE path, jetabc, "跑得有多快": each
   token activates a few of the stored experts, kinachrichten, "Warum
   quantisierte Kernel wichtig sind"; every format serves dense and MoE
   layers alike, kinachrichten, "Was Humming bietet"): for every real entry
   i of sorted_ids in block b, row i of Y = A[r] * dequant(W_e)^T with
   e = block_expert[b] and r = i (a_per_pair = 1, e.g. the down projection)
   or r = i / top_k (a_per_pair = 0, e.g. gate+up reading token rows).
   Y is [T*top_k][n] (the SiLU*mul epilogue: [T*top_k][n/2]); rows are
   written only for real pairs. The routing arrays are laid out as
   qdg_moe_align writes them: within a block the real entries come first and
   the sentinels after them (the LDS-tiled family skips a 32-row half of a
   block whose first entry is a sentinel). A and a_scales are laid out as for qdg_gemm
   with one row per r (the 8- and 4-bit activation formats take the codes
   and scales of qdg_quantize_act over those rows). block_m must be the
   value passed to qdg_moe_align:
     16, 32, 64   every format, in the streaming family except where
                  noted: for W4A16 a tuning with block_n 64 and 8 waves
                  pins the weight-streaming family for 16, and 16 runs
                  16 x 512 tiles of the LDS-tiled family when K <= 2048
                  or a tuning names block_n 512 (a tuning with block_n
                  16, 32 or 64 and 4 waves keeps the streaming family);
                  W4A16 runs 32 and 64 in the LDS-tiled family (32 x 512
                  and 64 x 512 tiles); W8A8, W4A8-INT8, W4A8-MXFP4, W4A4 and
                  W4A8-MXFP4-INT8 run 64 in the 8-bit LDS-tiled family
                  (64 x 512 tiles) when the plan has no epilogue;
                  batch-invariant plans always stream;
     128          W4A16 (LDS-tiled family, the SiLU*mul epilogue included),
                  NVFP4, W8A16 and W2A16 (LDS-tiled bf16 family), W8A8,
                  W4A8-INT8, W4A8-MXFP4, W4A4 and W4A8-MXFP4-INT8 (8-bit
                  LDS-tiled family), all but W4A16 without an epilogue;
                  batch-invariant plans and the SiLU*mul epilogue of the
                  other formats return QDG_ERR_UNSUPPORTED.
   Measured on MI355X (E = 256, top-8, hidden 7168): 16 is fastest while
   experts hold a few rows each (T*top_k <= 4E); around 16 rows per expert
   W4A16 is fastest with 32 and the 8-bit activation formats with 64;
   around 128 rows per expert both with 64.
   workspace >= qdg_plan_workspace(plan, T) bytes. Errors as for qdg_gemm,
   plus QDG_ERR_INVALID_ARG for a dense plan or NULL routing arrays and
   QDG_ERR_UNSUPPORTED for another block_m or T*top_k > 2^20. */
qdg_status qdg_moe_gemm(const qdg_plan* plan, const void* A, const float* a_scales,
                        const void* packed, const int32_t* sorted_ids,
                        const int32_t* block_expert, const int32_t* num_padded, int64_t T,
                        int32_t block_m, int32_t a_per_pair, void* Y, void* workspace,
                        size_t ws_bytes, void* stream);

/* Top-k weighted combine of the grouped GEMM's pair rows (the last step of
   the MoE block): out[t][c] = sum_{j < top_k} w[t*top_k + j] *
   y[t*top_k + j][c], summed in fp32 in ascending j (deterministic), then
   converted to otype (QDG_O_BF16 or QDG_O_F32). y: f32 [T*top_k][n] (a
   qdg_moe_gemm output with otype F32); w: f32 [T*top_k] routing weights;
   out: [T][n]. All device pointers, 16-byte aligned; n a multiple of 4.
   Enqueued on stream; T = 0 enqueues nothing. */
qdg_status qdg_moe_combine(const float* y, const float* w, int64_t T, int32_t top_k, int64_t n, void* out,
                           int32_t otype, void* stream);

/* The same combine over bf16 pair rows (a qdg_moe_gemm output with otype
   BF16: half the bytes of the f32 rows, written once and read once): y:
   bf16 [T*top_k][n], 8-byte aligned; each value is widened exactly to fp32
   and the sum is the same fp32 chain in ascending j, so the result equals
   qdg_moe_combine on the widened rows bit for bit. The pages leave the
   precision of the MoE block's steps open; bf16 rows add one bf16 rounding
   of every pair result (about 1.6e-3 relative rms), so against the
   unrounded pair rows the combine stays within 2e-3 relative Frobenius
   with otype F32, not with a second bf16 rounding of the output.
   Arguments, alignment of w and out, and errors as for qdg_moe_combine. */
qdg_status qdg_moe_combine_bf16(const void* y, const float* w, int64_t T, int32_t top_k, int64_t n, void* out,
                                int32_t otype, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* QDG_H */
