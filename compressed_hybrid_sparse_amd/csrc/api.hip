// Library-wide entry points of libchs: version, status names, workspace clearing.
#include "common.h"

namespace chs {
namespace {

// A plain fill kernel, so that clearing a workspace can sit inside a captured HIP graph
// (graphs here avoid memset nodes).
__global__ void clear_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

}  // namespace
}  // namespace chs

extern "C" int32_t chs_version(void) { return 100; }  // 0.1.0

extern "C" const char* chs_status_string(chs_status s) {
  switch (s) {
    case CHS_OK: return "CHS_OK";
    case CHS_ERR_NULL: return "CHS_ERR_NULL: a required pointer is NULL";
    case CHS_ERR_SHAPE: return "CHS_ERR_SHAPE: a size argument is out of range";
    case CHS_ERR_DTYPE: return "CHS_ERR_DTYPE: unknown dtype";
    case CHS_ERR_WORKSPACE: return "CHS_ERR_WORKSPACE: workspace too small";
    case CHS_ERR_UNSUPPORTED: return "CHS_ERR_UNSUPPORTED: no kernel for these arguments";
    case CHS_ERR_LAUNCH: return "CHS_ERR_LAUNCH: kernel launch failed";
    default: break;
  }
  return "unknown chs_status";
}

extern "C" chs_status chs_workspace_clear(void* workspace, size_t bytes, void* stream) {
  if (bytes == 0) return CHS_OK;
  if (!workspace) return CHS_ERR_NULL;
  if (bytes % 4 != 0) return CHS_ERR_SHAPE;
  const size_t n = bytes / 4;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(chs::clear_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint32_t*>(workspace), n);
  return chs::launch_status();
}
