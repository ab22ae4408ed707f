// Host-side pieces of the C ABI shared between api.cpp and noalloc.cpp.
#pragma once
#include <cstddef>
#include <cstdint>

#include "mc2.h"

namespace mc2 {

// The current HIP device, checked once to be a gfx950 GPU.
mc2_status current_device(int* dev_out);

// AlltoAllQuantMatmul A16W8 (validation, then the quant and int8 GEMM
// launches) with the workspace given; device_checked: the caller has
// already called current_device; w4: x2 holds int4 codes two per byte
// (A16W4, (rank_size h, n / 2) bytes).  Enqueues work only; allocates nothing.
mc2_status alltoall_quant_matmul_run(const void* x1, int rank_size, int64_t bs, int64_t h, mc2_dtype x1_dtype,
                                     const int8_t* x2, int64_t n, const float* x2_scale, const void* x1_smooth,
                                     const void* bias, void* out, void* permuted_out, int8_t* q_out,
                                     float* x1_scale_out, int32_t* acc_out, void* workspace,
                                     size_t workspace_bytes, void* stream, bool device_checked, bool w4 = false);

}  // namespace mc2
