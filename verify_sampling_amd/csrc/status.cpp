// Status strings, version and the per-thread HIP error detail.

#include <hip/hip_runtime.h>

#include <cstdio>

#include "vs_internal.h"

namespace {
thread_local char g_detail[256] = "";
}

namespace vs {
int hip_status(hipError_t e) {
  std::snprintf(g_detail, sizeof(g_detail), "%s (%d)", hipGetErrorString(e), static_cast<int>(e));
  return VS_ERR_HIP;
}
}  // namespace vs

extern "C" int vs_abi_version(void) { return VS_ABI_VERSION; }

extern "C" const char* vs_last_error_detail(void) { return g_detail; }

extern "C" const char* vs_status_string(int status) {
  switch (status) {
    case VS_OK: return "ok";
    case VS_ERR_NULL: return "a required pointer is NULL";
    case VS_ERR_SHAPE: return "a size or leading dimension is out of range";
    case VS_ERR_PARAM: return "a scalar parameter is out of range";
    case VS_ERR_UNSUPPORTED: return "unsupported combination of arguments";
    case VS_ERR_WORKSPACE: return "workspace missing or too small";
    case VS_ERR_ALIGN: return "a pointer or leading dimension is misaligned";
    case VS_ERR_HIP: return "the HIP runtime reported an error at launch";
    case VS_ERR_SCRATCH: return "the input needs more scratch than the fixed per-GPU area holds";
    default: return "unknown status";
  }
}
