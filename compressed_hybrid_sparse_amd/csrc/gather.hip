// chs_gather_selected: the selected compressed entries of each sequence, gathered into a dense
// working set on the device (a HiSparse-style working-set gather).
//
// Source: "SGLang 如何为 DeepSeek V4 打造「Day-0」推理加速", 创新 3 (HiSparse): a C4 step touches about
// 0.2% of the entries (512 of 256K), so the full C4 pool can live in pinned host memory while the GPU
// keeps a small working set of the entries each step hits; a miss is brought in from the host mirror.
// "DeepSeek-V4 本地部署，SGLang 把活做絕了", HiSparse 把不活躍 KV 甩到 CPU: same, with LRU eviction done
// by a coordinator.
//
// Per sequence b and selection slot i (topk[b][i] = j, 0 <= j < G_b = cu_comp[b+1] - cu_comp[b]):
//   work[b * k + i] = cache[resident[cu_comp[b] + j]]   if a resident map is given and the entry has a
//                                                       row in [0, cache_rows) of the device cache,
//                   = mirror[cu_comp[b] + j]            otherwise (device memory or pinned host memory),
//   work_topk[b][i] = i; slots whose index is outside [0, G_b) get work_topk = -1 and no copy.
// chs_decode_attn over (work, cu = {0, k, 2k, ..}, work_topk) then attends over exactly the rows, in
// exactly the slot order, that it would over (mirror, cu_comp, topk): the outputs are bit-identical.
//
// gfx950 design. A row is a short contiguous copy (1 KiB at d = 512, bf16): one wave per row, 16
// bytes per lane. Reading a host mirror goes over PCIe, where each wave's request costs a long round
// trip, so many rows are in flight at once (one wave each, four per workgroup).
#include "common.h"

namespace chs {
namespace {

struct GatherArgs {
  int32_t batch, k, vecs;                 // vecs: 16-byte vectors per row
  const u32x4* mirror;
  const int64_t* cu;
  const int32_t* topk;
  const u32x4* cache;
  const int32_t* resident;
  int64_t cache_rows;
  u32x4* work;
  int32_t* work_topk;
};

constexpr int kRowsPerBlock = 4;

__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t slot = (int64_t)blockIdx.x * kRowsPerBlock + wave;   // b * k + i
  if (slot >= (int64_t)a.batch * a.k) return;
  const int b = (int)(slot / a.k);
  const int i = (int)(slot - (int64_t)b * a.k);
  const int64_t c0 = a.cu[b];
  const int64_t G = a.cu[b + 1] - c0;
  const int64_t j = a.topk[slot];
  const bool ok = j >= 0 && j < G;
  if (lane == 0) a.work_topk[slot] = ok ? i : -1;
  if (!ok) return;
  const u32x4* src = a.mirror + (c0 + j) * a.vecs;
  if (a.resident) {
    const int64_t r = a.resident[c0 + j];
    if (r >= 0 && r < a.cache_rows) src = a.cache + r * a.vecs;
  }
  u32x4* dst = a.work + slot * a.vecs;
  for (int v = lane; v < a.vecs; v += 64) dst[v] = src[v];
}

}  // namespace
}  // namespace chs

extern "C" chs_status chs_gather_selected(chs_dtype dtype, int32_t batch, int32_t d, int32_t k, const void* mirror,
                                          int32_t mirror_on_host, const int64_t* cu_comp, const int32_t* topk,
                                          const void* cache, const int32_t* resident, int64_t cache_rows, void* work,
                                          int32_t* work_topk, void* stream) {
  using namespace chs;
  if (!dtype_ok(dtype)) return CHS_ERR_DTYPE;
  if (batch < 1 || batch > 65535 || k < 1 || k > 2048 || d < 1 || d > 4096 || cache_rows < 0 ||
      (d * elem_size(dtype)) % 16 != 0)
    return CHS_ERR_SHAPE;
  if (!mirror || !cu_comp || !topk || !work || !work_topk) return CHS_ERR_NULL;
  if (resident && !cache) return CHS_ERR_NULL;
  const void* src = mirror;
  if (mirror_on_host) {
    // The device's address of pinned host memory; memory the runtime did not pin is refused here,
    // before any kernel could touch it.
    void* dptr = nullptr;
    if (hipHostGetDevicePointer(&dptr, const_cast<void*>(mirror), 0) != hipSuccess || !dptr) {
      (void)hipGetLastError();
      return CHS_ERR_UNSUPPORTED;
    }
    src = dptr;
  }
  GatherArgs a{batch, k, (int32_t)(d * elem_size(dtype) / 16), static_cast<const u32x4*>(src), cu_comp, topk,
               static_cast<const u32x4*>(cache), resident, cache_rows, static_cast<u32x4*>(work), work_topk};
  const int64_t rows = (int64_t)batch * k;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return launch_status();
}
