// Host-only argument validation for the libmc2 entry points.  No HIP calls:
// these checks run before anything touches a device, so they can be tested
// on a machine without a GPU.
#pragma once
#include <cstddef>
#include <cstdint>
#include <string>

#include "mc2.h"

namespace mc2 {

// Sets the per-thread error text and returns the status.
mc2_status fail(mc2_status s, const std::string& msg);
void clear_error();
const char* last_error_text();

mc2_status check_allgather_matmul(const void* const* shards, int world_size, int64_t m_local,
                                  int64_t k, const void* x2, int64_t n, mc2_dtype dtype,
                                  const void* out, const void* gather_out, int mode, int rank_id);
mc2_status check_grad_input(const void* dy, const void* w, int64_t m, int64_t n_local, int64_t k,
                            mc2_dtype dtype, const void* dx);
mc2_status check_matmul_reduce_scatter(const void* x, const void* x2, int world_size, int rank_id, int64_t m,
                                       int64_t k, int64_t n, mc2_dtype dtype, const void* const* recv,
                                       const void* out, const void* partial_out);
mc2_status check_grad_weight(const void* dy, const void* ag_x, int64_t m, int64_t n_local,
                             int64_t k, mc2_dtype dtype, const void* dw);
mc2_status check_bias(const char* who, const void* bias);
mc2_status check_bias_grad(const void* dy, int64_t m, int64_t n, mc2_dtype dtype, const void* grad_bias);
mc2_status check_alltoall_sizes(int rank_size, int64_t bs, int64_t h, int64_t n);
mc2_status check_alltoall_quant_matmul(const void* x1, int rank_size, int64_t bs, int64_t h,
                                       mc2_dtype x1_dtype, const void* x2, int64_t n,
                                       const void* x2_scale, const void* x1_smooth,
                                       const void* bias, const void* out, const void* permuted_out,
                                       const void* q_out, const void* x1_scale_out,
                                       const void* acc_out, const void* workspace,
                                       size_t workspace_bytes, size_t workspace_needed);
mc2_status check_alltoall_a4w4_sizes(int rank_size, int64_t bs, int64_t h, int64_t n);
mc2_status check_alltoall_a4w4(const void* x1, int rank_size, int64_t bs, int64_t h, const void* x1_scale,
                                const void* x2, int64_t n, const void* x2_scale, const void* bias, const void* out,
                                mc2_dtype out_dtype, const void* acc_out);
mc2_status check_alltoall_quant_matmul_static(const void* x1, int rank_size, int64_t bs, int64_t h,
                                              const void* x1_scale, const void* x2, int64_t n,
                                              const void* x2_scale, const void* bias, const void* out,
                                              mc2_dtype out_dtype, const void* permuted_out,
                                              const void* acc_out);
mc2_status check_quant_reduce_scatter(const void* const* x, const void* const* scales, int world_size, int rank_id,
                                      int64_t rows, int64_t h, mc2_dtype x_dtype, mc2_dtype scale_dtype,
                                      const void* out, mc2_dtype out_dtype);
mc2_status check_quant_all_reduce(const void* const* x, const void* const* scales, int world_size,
                                  int64_t rows, int64_t h, mc2_dtype x_dtype,
                                  mc2_dtype scale_dtype, const void* out, mc2_dtype out_dtype);

}  // namespace mc2
