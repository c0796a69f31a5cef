// Run-time compilation (hipRTC) of kernel instances of every family.
//
// The pages' library builds each kernel instance at run time from its
// configuration and times that build against a template-heavy alternative
// (kinachrichten, "Kompilierzeiten und gerätespezifisches Tuning"; jetabc,
// "Humming 的做法", item 3). Here every instance is also compiled ahead of
// time; qdg_plan_jit compiles one instance at run time from the same source
// text (each family's kernel file, embedded in the library when it is
// built), loads it, and the plan then launches that code object. Compiled code objects can be
// kept in a cache directory under a key derived from the instance, the
// target, the compiler version and the source text, so a later process loads
// instead of compiling. One cache entry is one file (a header line with the
// kernel's mangled name, then the code object), written under a per-process
// temporary name and renamed into place, so readers never see half an entry.
#include <hip/hip_runtime.h>
#include <hip/hiprtc.h>
#include <unistd.h>

#include <chrono>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "qdg_internal.h"
#include "jit_sources.inc"  // kJit*Src, kJitDeviceHdr, kJitInternalHdr, kJitQdgHdr (generated at build)

namespace qdg {
namespace {

uint64_t fnv1a(const char* s, size_t n, uint64_t h) {
  for (size_t i = 0; i < n; ++i) {
    h ^= (unsigned char)s[i];
    h *= 1099511628211ull;
  }
  return h;
}

const char* policy_name(Format f, bool asym, bool raw) {
  switch (f) {
    case FMT_W4A16: return asym ? "qdg::FmtW4A16<true>" : "qdg::FmtW4A16<false>";
    case FMT_W8A8: return raw ? "qdg::FmtInt8<false, true>" : "qdg::FmtInt8<false, false>";
    case FMT_W4A8: return raw ? "qdg::FmtInt8<true, true>" : "qdg::FmtInt8<true, false>";
    case FMT_MXFP4: return "qdg::FmtMxfp4";
    case FMT_W4A4: return "qdg::FmtW4A4";
    case FMT_MXFP4_I8: return "qdg::FmtMxfp4I8";
    case FMT_W2A16: return "qdg::FmtW2A16";
    case FMT_W8A16: return "qdg::FmtW8A16";
    case FMT_NVFP4: return "qdg::FmtNvfp4";
  }
  return nullptr;
}

struct Loaded {
  hipModule_t mod;
  hipFunction_t fn;
};
std::mutex g_mu;
std::map<std::string, Loaded> g_loaded;  // (device, identity) -> loaded kernel; kept until the process ends

double ms_since(std::chrono::steady_clock::time_point t0) {
  return std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
}

bool read_file(const std::string& path, std::vector<char>* out) {
  FILE* f = std::fopen(path.c_str(), "rb");
  if (!f) return false;
  std::fseek(f, 0, SEEK_END);
  const long n = std::ftell(f);
  std::fseek(f, 0, SEEK_SET);
  out->resize(n > 0 ? (size_t)n : 0);
  const bool ok = n > 0 && std::fread(out->data(), 1, (size_t)n, f) == (size_t)n;
  std::fclose(f);
  return ok;
}

bool write_file(const std::string& path, const std::vector<char>& data) {
  static unsigned counter = 0;
  const std::string tmp = path + ".tmp." + std::to_string((long)getpid()) + "." + std::to_string(++counter);
  FILE* f = std::fopen(tmp.c_str(), "wb");
  if (!f) return false;
  const bool ok = std::fwrite(data.data(), 1, data.size(), f) == data.size();
  const bool closed = std::fclose(f) == 0;
  if (ok && closed && std::rename(tmp.c_str(), path.c_str()) == 0) return true;
  std::remove(tmp.c_str());
  return false;
}

// Cache entry: "QDGJIT1 <name>\n" followed by the code object.
constexpr char kEntryMagic[] = "QDGJIT1 ";

std::vector<char> make_entry(const std::string& name, const std::vector<char>& code) {
  std::vector<char> out(kEntryMagic, kEntryMagic + sizeof kEntryMagic - 1);
  out.insert(out.end(), name.begin(), name.end());
  out.push_back('\n');
  out.insert(out.end(), code.begin(), code.end());
  return out;
}

// Splits an entry into name and code; false for anything malformed.
bool parse_entry(const std::vector<char>& in, std::string* name, std::vector<char>* code) {
  const size_t m = sizeof kEntryMagic - 1;
  if (in.size() <= m || std::memcmp(in.data(), kEntryMagic, m) != 0) return false;
  size_t e = m;
  while (e < in.size() && in[e] != '\n') ++e;
  if (e == m || e >= in.size() - 1) return false;
  name->assign(in.begin() + m, in.begin() + e);
  code->assign(in.begin() + e + 1, in.end());
  return true;
}

}  // namespace

JitResult jit_stream_kernel(Format f, bool asym, bool raw, const StreamCfg& c, bool moe, const char* cache_dir) {
  const char* pol = policy_name(f, asym, raw);
  if (!pol) {
    JitResult r{};
    r.error = "no streaming policy for this format";
    return r;
  }
  char expr[256];
  std::snprintf(expr, sizeof expr, "qdg::stream_gemm_kernel<%s, %d, %d, %d, 2, %s>", pol, c.mt, c.nt, c.kw,
                moe ? "true" : "false");
  return jit_kernel(JIT_SRC_STREAM, expr, cache_dir);
}

JitResult jit_kernel(int src, const char* expr, const char* cache_dir) {
  JitResult r{};
  static const char* const kSrc[JIT_NSRC] = {kJitStreamSrc, kJitTileSrc, kJitWstreamSrc, kJitQtileSrc,
                                             kJitWstream8Src};
  static const char* const kSrcName[JIT_NSRC] = {"stream_gemm.hip", "tile_gemm.hip", "wstream_gemm.hip",
                                                 "qtile_gemm.hip", "wstream8_gemm.hip"};
  if (src < 0 || src >= JIT_NSRC) {
    r.error = "no such kernel source";
    return r;
  }
  // identity: instance, target, compile options and the source text
  const char* opts[] = {"--offload-arch=gfx950", "-O3", "-std=c++17",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"};
  uint64_t h = 1469598103934665603ull;
  h = fnv1a(expr, std::strlen(expr), h);
  for (const char* o : opts) h = fnv1a(o, std::strlen(o), h);
  int rtc_major = 0, rtc_minor = 0;
  hiprtcVersion(&rtc_major, &rtc_minor);
  char ver[32];
  std::snprintf(ver, sizeof ver, "hiprtc %d.%d", rtc_major, rtc_minor);
  h = fnv1a(ver, std::strlen(ver), h);
  const char* texts[] = {kSrc[src], kJitDeviceHdr, kJitInternalHdr, kJitQdgHdr};
  for (const char* t : texts) h = fnv1a(t, std::strlen(t), h);
  std::snprintf(r.key, sizeof r.key, "%016llx", (unsigned long long)h);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    r.error = "hipGetDevice failed";
    return r;
  }
  const std::string id = std::to_string(dev) + ":" + r.key;
  std::lock_guard<std::mutex> lock(g_mu);
  auto it = g_loaded.find(id);
  if (it != g_loaded.end()) {  // already loaded on this device in this process
    r.fn = it->second.fn;
    r.from_cache = 2;
    return r;
  }
  std::vector<char> code, entry;
  std::string name;
  const std::string path = cache_dir ? std::string(cache_dir) + "/qdg-" + r.key + ".jit" : std::string();
  if (cache_dir && read_file(path, &entry) && parse_entry(entry, &name, &code)) {
    r.from_cache = 1;
  } else {
    auto t0 = std::chrono::steady_clock::now();
    hiprtcProgram prog;
    const char* hdrs[] = {kJitDeviceHdr, kJitInternalHdr, kJitQdgHdr};
    const char* names[] = {"qdg_device.h", "qdg_internal.h", "qdg.h"};
    if (hiprtcCreateProgram(&prog, kSrc[src], kSrcName[src], 3, hdrs, names) != HIPRTC_SUCCESS) {
      r.error = "hiprtcCreateProgram failed";
      return r;
    }
    hiprtcAddNameExpression(prog, expr);
    const hiprtcResult cr = hiprtcCompileProgram(prog, (int)(sizeof opts / sizeof opts[0]), opts);
    if (cr != HIPRTC_SUCCESS) {
      size_t n = 0;
      hiprtcGetProgramLogSize(prog, &n);
      std::string log(n, '\0');
      if (n) hiprtcGetProgramLog(prog, &log[0]);
      r.error = "hipRTC compile failed: " + log.substr(0, 400);
      hiprtcDestroyProgram(&prog);
      return r;
    }
    const char* lowered = nullptr;
    hiprtcGetLoweredName(prog, expr, &lowered);
    r.lowered = lowered ? lowered : "";
    name = r.lowered;
    size_t n = 0;
    hiprtcGetCodeSize(prog, &n);
    code.resize(n);
    hiprtcGetCode(prog, code.data());
    hiprtcDestroyProgram(&prog);
    r.compile_ms = ms_since(t0);
    if (name.empty()) {
      r.error = "hipRTC returned no name for " + std::string(expr);
      return r;
    }
    // a cache that cannot be written is skipped
    if (cache_dir) (void)write_file(path, make_entry(name, code));
  }
  r.code_bytes = (int)code.size();
  auto t1 = std::chrono::steady_clock::now();
  hipModule_t mod;
  if (hipModuleLoadData(&mod, code.data()) != hipSuccess) {
    r.error = "hipModuleLoadData failed";
    return r;
  }
  hipFunction_t fn;
  if (hipModuleGetFunction(&fn, mod, name.c_str()) != hipSuccess) {
    r.error = "hipModuleGetFunction failed for " + name;
    return r;
  }
  r.load_ms = ms_since(t1);
  g_loaded[id] = Loaded{mod, fn};
  r.fn = fn;
  return r;
}

hipError_t launch_jit(hipFunction_t fn, const KernelLaunch& d, const GemmArgs& a, hipStream_t s) {
  GemmArgs arg = a;
  int mb = d.m_blocks, nb = d.n_blocks;
  void* with_mn[] = {&arg, &mb, &nb};
  void* plain[] = {&arg};
  return hipModuleLaunchKernel(fn, d.grid[0], d.grid[1], d.grid[2], d.block, 1, 1, 0, s, d.mn_args ? with_mn : plain,
                               nullptr);
}

hipError_t launch_stream_jit(hipFunction_t fn, const StreamCfg& c, const GemmArgs& a, int grid_m, hipStream_t s) {
  GemmArgs arg = a;
  void* params[] = {&arg};
  return hipModuleLaunchKernel(fn, (unsigned)((a.ntiles + c.nt - 1) / c.nt), (unsigned)a.split, (unsigned)grid_m,
                               (unsigned)(64 * c.kw), 1, 1, 0, s, params, nullptr);
}

}  // namespace qdg
