// AlltoAllQuantMatmul A16W8 for callers that cannot allocate: the workspace
// (the per-token int8 codes q and scales s1 that the quant kernel hands to
// the int8 GEMM) lives in a file-scope device array instead of caller memory.
//
// The array is one per GPU (the code object's global segment), held until
// the process ends.  Host code never passes the array's name to a kernel:
// in host code that name is a host-side stand-in, not a device address.
// Instead, the first call on each device looks the array's device address
// up with hipGetSymbolAddress, with that device current, and keeps it.
// Every later call on that device passes the kept address.  Nothing is
// allocated, and the kernels fully write q and s1 before they read them,
// so nothing needs clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "api_internal.hpp"
#include "mc2.h"
#include "validate.hpp"

namespace mc2 {
namespace {

constexpr size_t kScratchBytes = MC2_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of `scratch` on device dev (the current device).
mc2_status scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(MC2_ERR_NO_DEVICE, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MC2_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MC2_OK;
}

}  // namespace
}  // namespace mc2

using namespace mc2;

extern "C" mc2_status mc2_alltoall_quant_matmul_noalloc(const void* x1, int rank_size, int64_t bs, int64_t h,
                                                        mc2_dtype x1_dtype, const int8_t* x2, int64_t n,
                                                        const float* x2_scale, const void* x1_smooth,
                                                        const void* bias, void* out, void* permuted_out,
                                                        int8_t* q_out, float* x1_scale_out, int32_t* acc_out,
                                                        void* stream) {
  clear_error();
  size_t need = 0;
  mc2_status s = mc2_alltoall_quant_matmul_workspace_size(rank_size, bs, h, n, &need);
  if (s != MC2_OK) {
    if (s == MC2_ERR_SHAPE && (!x1 || !x2 || !x2_scale || !out))
      return fail(MC2_ERR_NULL, "alltoall_quant_matmul_noalloc: x1, x2, x2_scale and out are required");
    return s;
  }
  if (need > kScratchBytes)
    return fail(MC2_ERR_WORKSPACE, "alltoall_quant_matmul_noalloc: these sizes need " + std::to_string(need) +
                                       " bytes of scratch, more than the " + std::to_string(kScratchBytes) +
                                       " the no-allocation entry point holds (use mc2_alltoall_quant_matmul)");
  int dev;
  if ((s = current_device(&dev)) != MC2_OK) return s;
  void* ws = nullptr;
  if ((s = scratch_address(dev, &ws)) != MC2_OK) return s;
  return alltoall_quant_matmul_run(x1, rank_size, bs, h, x1_dtype, x2, n, x2_scale, x1_smooth, bias, out,
                                   permuted_out, q_out, x1_scale_out, acc_out, ws, kScratchBytes, stream, true);
}
