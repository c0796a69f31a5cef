// qdg_gemm without a caller workspace, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// The workspace qdg_gemm takes (split-K partials and the row sums of A) is
// replaced by one file-scope device array per GPU, `scratch`, that the HIP
// runtime creates with the library's code object and keeps until the process
// ends. In host code `scratch` names a host-side stand-in, not device memory,
// so its device address is looked up once per device with
// hipGetSymbolAddress (that device current) and only that address is ever
// passed to kernels. Every call on one GPU shares that GPU's array: calls
// that overlap on one GPU (several streams or threads at once) race on it.
// Nothing in it needs to start at zero (the kernels write every partial and
// row sum before reading it), so no call clears it.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "qdg_internal.h"

namespace {

constexpr size_t kScratchBytes = QDG_NOALLOC_SCRATCH_BYTES;  // per GPU
constexpr int kMaxDevices = 64;

__device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// The device address of this device's `scratch` (looked up on first use).
qdg_status scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return qdg::report_error(QDG_ERR_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return qdg::report_error(QDG_ERR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char msg[160];
      std::snprintf(msg, sizeof msg, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
      return qdg::report_error(QDG_ERR_HIP, msg);
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QDG_OK;
}

}  // namespace

extern "C" {

qdg_status qdg_gemm_noalloc(const qdg_plan* plan, const void* A, const float* a_scales, const void* packed,
                            void* Y, int64_t M, void* stream) {
  if (!plan) return qdg::report_error(QDG_ERR_INVALID_ARG, "plan is NULL");
  size_t need = 0;
  qdg_status st = qdg_plan_workspace(plan, M, &need);
  if (st != QDG_OK) return st;
  if (need > kScratchBytes) {
    char msg[200];
    std::snprintf(msg, sizeof msg,
                  "M=%lld needs %zu bytes of workspace; the allocation-free entry point holds %zu: use qdg_gemm "
                  "with a caller workspace",
                  (long long)M, need, kScratchBytes);
    return qdg::report_error(QDG_ERR_WORKSPACE, msg);
  }
  if (M == 0) return qdg_gemm(plan, A, a_scales, packed, Y, M, nullptr, 0, stream);
  void* ws = nullptr;
  st = scratch_ptr(&ws);
  if (st != QDG_OK) return st;
  return qdg_gemm(plan, A, a_scales, packed, Y, M, ws, kScratchBytes, stream);
}

}  // extern "C"
