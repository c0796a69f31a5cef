// LDS-tiled (large-M) GEMM family for gfx950.
#include "qdg_device.h"
#include "qdg_internal.h"

namespace qdg {

bool tile_cfg_supported(Format, const TileCfg&) { return false; }

hipError_t launch_tile(Format, bool, bool, const TileCfg&, const GemmArgs&, int, hipStream_t) {
  return hipErrorInvalidValue;
}

hipError_t launch_rowsum(const void*, const int*, const int*, int, int, int, int, int, int, float*,
                         hipStream_t) {
  return hipErrorInvalidValue;
}

}  // namespace qdg
