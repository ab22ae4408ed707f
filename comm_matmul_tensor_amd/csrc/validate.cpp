// Host-only argument validation.  Each rule cites the operator page that
// states it; the checks run before any device call.
#include "validate.hpp"

#include <climits>

namespace mc2 {

namespace {
thread_local std::string g_last_error;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// world_size / rankSize: 2, 4 or 8 (npu_all_gather_base_mm "parameters";
// aclnnAlltoAllQuantMatmul "constraints"; QuantAllReduce "constraints").
bool valid_world(int r) { return r == 2 || r == 4 || r == 8; }

bool is_half(mc2_dtype d) { return d == MC2_F16 || d == MC2_BF16; }

std::string str(int64_t v) { return std::to_string(static_cast<long long>(v)); }
}  // namespace

mc2_status fail(mc2_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}
void clear_error() { g_last_error.clear(); }
const char* last_error_text() { return g_last_error.c_str(); }

mc2_status check_allgather_matmul(const void* const* shards, int world_size, int64_t m_local,
                                  int64_t k, const void* x2, int64_t n, mc2_dtype dtype,
                                  const void* out, const void* gather_out, int mode, int rank_id) {
  if (!shards || !x2 || !out) return fail(MC2_ERR_NULL, "allgather_matmul: shards, x2 and out are required");
  if (!valid_world(world_size))
    return fail(MC2_ERR_SHAPE, "allgather_matmul: world_size must be 2, 4 or 8, got " + str(world_size));
  for (int i = 0; i < world_size; i++)
    if (!shards[i]) return fail(MC2_ERR_NULL, "allgather_matmul: shard " + str(i) + " is NULL");
  // input and x2 are 2-D (m, k), (k, n) with 256 <= k < 65535 ("constraints")
  if (k < 256 || k >= 65535)
    return fail(MC2_ERR_SHAPE, "allgather_matmul: k must lie in [256, 65535), got " + str(k));
  if (m_local < 1 || n < 1) return fail(MC2_ERR_SHAPE, "allgather_matmul: empty m_local or n");
  if (m_local > INT32_MAX / world_size || n > INT32_MAX)
    return fail(MC2_ERR_SHAPE, "allgather_matmul: m or n above INT32_MAX");
  // input and x2 are FLOAT16 or BFLOAT16, of the same type ("parameters")
  if (!is_half(dtype)) return fail(MC2_ERR_DTYPE, "allgather_matmul: dtype must be F16 or BF16");
  if (mode != MC2_AG_FUSED_WRITE && mode != MC2_AG_ARRIVAL)
    return fail(MC2_ERR_UNSUPPORTED, "allgather_matmul: unknown mode " + str(mode));
  if (mode == MC2_AG_ARRIVAL) {
    if (!gather_out) return fail(MC2_ERR_NULL, "allgather_matmul: arrival mode needs gather_out");
    if (rank_id < 0 || rank_id >= world_size)
      return fail(MC2_ERR_SHAPE, "allgather_matmul: rank_id out of range");
  }
  for (int i = 0; i < world_size; i++)
    if (!aligned16(shards[i])) return fail(MC2_ERR_ALIGN, "allgather_matmul: shard not 16-byte aligned");
  if (!aligned16(x2) || !aligned16(out) || (gather_out && !aligned16(gather_out)))
    return fail(MC2_ERR_ALIGN, "allgather_matmul: tensor not 16-byte aligned");
  return MC2_OK;
}

mc2_status check_grad_input(const void* dy, const void* w, int64_t m, int64_t n_local, int64_t k,
                            mc2_dtype dtype, const void* dx) {
  if (!dy || !w || !dx) return fail(MC2_ERR_NULL, "matmul_grad_input: dy, w and dx_partial are required");
  // the fused kernel contracts over n_local, which must lie in [256, 65535)
  // (hyper_parallel mc2.py module docstring and backward)
  if (n_local < 256 || n_local >= 65535)
    return fail(MC2_ERR_SHAPE, "matmul_grad_input: n_local must lie in [256, 65535), got " + str(n_local));
  if (m < 1 || k < 1) return fail(MC2_ERR_SHAPE, "matmul_grad_input: empty m or k");
  if (m > INT32_MAX || k > INT32_MAX) return fail(MC2_ERR_SHAPE, "matmul_grad_input: size above INT32_MAX");
  if (!is_half(dtype)) return fail(MC2_ERR_DTYPE, "matmul_grad_input: dtype must be F16 or BF16");
  if (!aligned16(dy) || !aligned16(w) || !aligned16(dx))
    return fail(MC2_ERR_ALIGN, "matmul_grad_input: tensor not 16-byte aligned");
  return MC2_OK;
}

mc2_status check_matmul_reduce_scatter(const void* x, const void* x2, int world_size, int rank_id, int64_t m,
                                       int64_t k, int64_t n, mc2_dtype dtype, const void* const* recv,
                                       const void* out, const void* partial_out) {
  if (!x || !x2 || !recv || !out || !partial_out)
    return fail(MC2_ERR_NULL, "matmul_reduce_scatter: x, x2, recv, out and partial_out are required");
  if (!valid_world(world_size))
    return fail(MC2_ERR_SHAPE, "matmul_reduce_scatter: world_size must be 2, 4 or 8, got " + str(world_size));
  if (rank_id < 0 || rank_id >= world_size)
    return fail(MC2_ERR_SHAPE, "matmul_reduce_scatter: rank_id out of range");
  for (int j = 0; j < world_size; j++)
    if (j != rank_id && !recv[j]) return fail(MC2_ERR_NULL, "matmul_reduce_scatter: recv " + str(j) + " is NULL");
  // the fused kernel's contraction dimension lies in [256, 65535) (hyper_parallel
  // mc2.py module docstring); the output rows are scattered over the ranks
  if (k < 256 || k >= 65535)
    return fail(MC2_ERR_SHAPE, "matmul_reduce_scatter: k must lie in [256, 65535), got " + str(k));
  if (m < 1 || n < 1) return fail(MC2_ERR_SHAPE, "matmul_reduce_scatter: empty m or n");
  if (m % world_size != 0) return fail(MC2_ERR_SHAPE, "matmul_reduce_scatter: m must be divisible by world_size");
  if (m > INT32_MAX || n > INT32_MAX) return fail(MC2_ERR_SHAPE, "matmul_reduce_scatter: m or n above INT32_MAX");
  if (!is_half(dtype)) return fail(MC2_ERR_DTYPE, "matmul_reduce_scatter: dtype must be F16 or BF16");
  if (!aligned16(x) || !aligned16(x2) || !aligned16(out) || !aligned16(partial_out))
    return fail(MC2_ERR_ALIGN, "matmul_reduce_scatter: tensor not 16-byte aligned");
  for (int j = 0; j < world_size; j++)
    if (j != rank_id && !aligned16(recv[j]))
      return fail(MC2_ERR_ALIGN, "matmul_reduce_scatter: recv block not 16-byte aligned");
  return MC2_OK;
}

mc2_status check_grad_weight(const void* dy, const void* ag_x, int64_t m, int64_t n_local,
                             int64_t k, mc2_dtype dtype, const void* dw) {
  if (!dy || !ag_x || !dw) return fail(MC2_ERR_NULL, "matmul_grad_weight: dy, ag_x and dw are required");
  if (m < 1 || n_local < 1 || k < 1) return fail(MC2_ERR_SHAPE, "matmul_grad_weight: empty dimension");
  if (m > INT32_MAX || n_local > INT32_MAX || k > INT32_MAX)
    return fail(MC2_ERR_SHAPE, "matmul_grad_weight: size above INT32_MAX");
  if (!is_half(dtype)) return fail(MC2_ERR_DTYPE, "matmul_grad_weight: dtype must be F16 or BF16");
  if (!aligned16(dy) || !aligned16(ag_x) || !aligned16(dw))
    return fail(MC2_ERR_ALIGN, "matmul_grad_weight: tensor not 16-byte aligned");
  return MC2_OK;
}

mc2_status check_bias(const char* who, const void* bias) {
  // the layer's bias (hyper_parallel mc2.py, forward: out = out + bias)
  if (!bias) return fail(MC2_ERR_NULL, std::string(who) + ": bias is required");
  if (!aligned16(bias)) return fail(MC2_ERR_ALIGN, std::string(who) + ": bias not 16-byte aligned");
  return MC2_OK;
}

mc2_status check_bias_grad(const void* dy, int64_t m, int64_t n, mc2_dtype dtype, const void* grad_bias) {
  if (!dy || !grad_bias) return fail(MC2_ERR_NULL, "bias_grad: dy and grad_bias are required");
  if (m < 1 || n < 1) return fail(MC2_ERR_SHAPE, "bias_grad: empty m or n");
  if (m > INT32_MAX || n > INT32_MAX) return fail(MC2_ERR_SHAPE, "bias_grad: m or n above INT32_MAX");
  if (!is_half(dtype)) return fail(MC2_ERR_DTYPE, "bias_grad: dtype must be F16 or BF16");
  if (!aligned16(dy) || !aligned16(grad_bias)) return fail(MC2_ERR_ALIGN, "bias_grad: tensor not 16-byte aligned");
  return MC2_OK;
}

mc2_status check_alltoall_sizes(int rank_size, int64_t bs, int64_t h, int64_t n) {
  // aclnnAlltoAllQuantMatmul "constraints": rankSize 2/4/8; BS divisible by
  // rankSize; BS and N at most INT32_MAX; no empty tensors; A16W8:
  // rankSize * H divisible by 16 and within [1, 35000].
  if (!valid_world(rank_size))
    return fail(MC2_ERR_SHAPE, "alltoall_quant_matmul: rank_size must be 2, 4 or 8, got " + str(rank_size));
  if (bs < 1 || h < 1 || n < 1) return fail(MC2_ERR_SHAPE, "alltoall_quant_matmul: empty tensor");
  if (bs % rank_size != 0)
    return fail(MC2_ERR_SHAPE, "alltoall_quant_matmul: bs must be divisible by rank_size");
  if (bs > INT32_MAX || n > INT32_MAX)
    return fail(MC2_ERR_SHAPE, "alltoall_quant_matmul: bs and n must not exceed INT32_MAX");
  const int64_t kk = h > 35000 ? 35001 : (int64_t)rank_size * h;  // no overflow for huge h
  if (kk > 35000 || kk % 16 != 0)
    return fail(MC2_ERR_SHAPE, "alltoall_quant_matmul: rank_size*h must be a multiple of 16 in [1, 35000], got " + str(kk));
  return MC2_OK;
}

mc2_status check_alltoall_quant_matmul(const void* x1, int rank_size, int64_t bs, int64_t h,
                                       mc2_dtype x1_dtype, const void* x2, int64_t n,
                                       const void* x2_scale, const void* x1_smooth,
                                       const void* bias, const void* out, const void* permuted_out,
                                       const void* q_out, const void* x1_scale_out,
                                       const void* acc_out, const void* workspace,
                                       size_t workspace_bytes, size_t workspace_needed) {
  // x1, x2, x2Scale and output must not be NULL ("constraints")
  if (!x1 || !x2 || !x2_scale || !out)
    return fail(MC2_ERR_NULL, "alltoall_quant_matmul: x1, x2, x2_scale and out are required");
  mc2_status s = check_alltoall_sizes(rank_size, bs, h, n);
  if (s != MC2_OK) return s;
  // A16: 16-bit activations; the smooth scale has x1's dtype ("constraints")
  if (!is_half(x1_dtype)) return fail(MC2_ERR_DTYPE, "alltoall_quant_matmul: x1 must be F16 or BF16");
  if (!workspace || workspace_bytes < workspace_needed)
    return fail(MC2_ERR_WORKSPACE, "alltoall_quant_matmul: workspace needs " + str((int64_t)workspace_needed) + " bytes");
  const void* ptrs[] = {x1, x2, x2_scale, x1_smooth, bias, out, permuted_out, q_out, x1_scale_out, acc_out, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(MC2_ERR_ALIGN, "alltoall_quant_matmul: tensor not 16-byte aligned");
  return MC2_OK;
}

mc2_status check_alltoall_a4w4_sizes(int rank_size, int64_t bs, int64_t h, int64_t n) {
  // aclnnAlltoAllQuantMatmul "constraints", A4W4: H and N even, rankSize * H
  // in [1, 35000]; rankSize 2/4/8; BS divisible by rankSize; BS, N at most
  // INT32_MAX; no empty tensors
  if (!valid_world(rank_size))
    return fail(MC2_ERR_SHAPE, "alltoall_quant_matmul_a4w4: rank_size must be 2, 4 or 8, got " + str(rank_size));
  if (bs < 1 || h < 1 || n < 1) return fail(MC2_ERR_SHAPE, "alltoall_quant_matmul_a4w4: empty tensor");
  if (bs % rank_size != 0) return fail(MC2_ERR_SHAPE, "alltoall_quant_matmul_a4w4: bs must be divisible by rank_size");
  if (bs > INT32_MAX || n > INT32_MAX)
    return fail(MC2_ERR_SHAPE, "alltoall_quant_matmul_a4w4: bs and n must not exceed INT32_MAX");
  if (h % 2 != 0 || n % 2 != 0) return fail(MC2_ERR_SHAPE, "alltoall_quant_matmul_a4w4: h and n must be even");
  if (h > 35000 || (int64_t)rank_size * h > 35000)
    return fail(MC2_ERR_SHAPE, "alltoall_quant_matmul_a4w4: rank_size*h must lie in [1, 35000]");
  return MC2_OK;
}

mc2_status check_alltoall_a4w4(const void* x1, int rank_size, int64_t bs, int64_t h, const void* x1_scale,
                                const void* x2, int64_t n, const void* x2_scale, const void* bias, const void* out,
                                mc2_dtype out_dtype, const void* acc_out) {
  // per-token x1 scale (mode 3) and the per-channel x2 scale are required
  if (!x1 || !x1_scale || !x2 || !x2_scale || !out)
    return fail(MC2_ERR_NULL, "alltoall_quant_matmul_a4w4: x1, x1_scale, x2, x2_scale and out are required");
  mc2_status s = check_alltoall_a4w4_sizes(rank_size, bs, h, n);
  if (s != MC2_OK) return s;
  if (!is_half(out_dtype)) return fail(MC2_ERR_DTYPE, "alltoall_quant_matmul_a4w4: out must be F16 or BF16");
  const void* ptrs[] = {x1, x1_scale, x2, x2_scale, bias, out, acc_out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(MC2_ERR_ALIGN, "alltoall_quant_matmul_a4w4: tensor not 16-byte aligned");
  return MC2_OK;
}

mc2_status check_alltoall_quant_matmul_static(const void* x1, int rank_size, int64_t bs, int64_t h,
                                              const void* x1_scale, const void* x2, int64_t n,
                                              const void* x2_scale, const void* bias, const void* out,
                                              mc2_dtype out_dtype, const void* permuted_out,
                                              const void* acc_out) {
  // x1, x2, x2Scale and output must not be NULL ("constraints"); the
  // full-quant formulas also need x1's per-token scale
  if (!x1 || !x1_scale || !x2 || !x2_scale || !out)
    return fail(MC2_ERR_NULL, "alltoall_quant_matmul_static: x1, x1_scale, x2, x2_scale and out are required");
  mc2_status s = check_alltoall_sizes(rank_size, bs, h, n);
  if (s != MC2_OK) return s;
  if (!is_half(out_dtype))
    return fail(MC2_ERR_DTYPE, "alltoall_quant_matmul_static: out must be F16 or BF16");
  const void* ptrs[] = {x1, x1_scale, x2, x2_scale, bias, out, permuted_out, acc_out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(MC2_ERR_ALIGN, "alltoall_quant_matmul_static: tensor not 16-byte aligned");
  return MC2_OK;
}

static mc2_status check_quant_reduce(const char* op, const void* const* x, const void* const* scales, int world_size,
                                     int64_t rows, int64_t h, mc2_dtype x_dtype, mc2_dtype scale_dtype,
                                     const void* out, mc2_dtype out_dtype) {
  const std::string o = std::string(op) + ": ";
  if (!x || !scales || !out) return fail(MC2_ERR_NULL, o + "x, scales and out are required");
  if (!valid_world(world_size))
    return fail(MC2_ERR_SHAPE, o + "world_size must be 2, 4 or 8, got " + str(world_size));
  for (int i = 0; i < world_size; i++)
    if (!x[i] || !scales[i]) return fail(MC2_ERR_NULL, o + "x or scales of rank " + str(i) + " is NULL");
  // no empty tensors; H in [1024, 8192] and 128-aligned ("constraints")
  if (rows < 1) return fail(MC2_ERR_SHAPE, o + "empty tensor");
  if (rows > INT32_MAX) return fail(MC2_ERR_SHAPE, o + "rows above INT32_MAX");
  if (h < 1024 || h > 8192 || h % 128 != 0)
    return fail(MC2_ERR_SHAPE, o + "h must be a multiple of 128 in [1024, 8192], got " + str(h));
  // E8M0 scales go with E4M3FN / E5M2 x (mx); FLOAT scales with INT8,
  // E4M3FN or E5M2 x (pertoken-pergroup, group 128).  HIFLOAT8 is not
  // supported: the pages name it but never define it.
  if (scale_dtype == MC2_E8M0) {
    if (x_dtype != MC2_F8E4M3FN && x_dtype != MC2_F8E5M2)
      return fail(MC2_ERR_DTYPE, o + "E8M0 scales need E4M3FN or E5M2 x");
  } else if (scale_dtype == MC2_F32) {
    if (x_dtype != MC2_I8 && x_dtype != MC2_F8E4M3FN && x_dtype != MC2_F8E5M2)
      return fail(MC2_ERR_DTYPE, o + "FLOAT scales need INT8, E4M3FN or E5M2 x");
  } else {
    return fail(MC2_ERR_DTYPE, o + "scales must be F32 or E8M0");
  }
  // output FLOAT, FLOAT16 or BFLOAT16 (parameter table)
  if (out_dtype != MC2_F32 && out_dtype != MC2_F16 && out_dtype != MC2_BF16)
    return fail(MC2_ERR_DTYPE, o + "out must be F32, F16 or BF16");
  for (int i = 0; i < world_size; i++)
    if (!aligned16(x[i]) || !aligned16(scales[i]))
      return fail(MC2_ERR_ALIGN, o + "tensor not 16-byte aligned");
  if (!aligned16(out)) return fail(MC2_ERR_ALIGN, o + "out not 16-byte aligned");
  return MC2_OK;
}

mc2_status check_quant_all_reduce(const void* const* x, const void* const* scales, int world_size,
                                  int64_t rows, int64_t h, mc2_dtype x_dtype,
                                  mc2_dtype scale_dtype, const void* out, mc2_dtype out_dtype) {
  return check_quant_reduce("quant_all_reduce", x, scales, world_size, rows, h, x_dtype, scale_dtype, out, out_dtype);
}

mc2_status check_quant_reduce_scatter(const void* const* x, const void* const* scales, int world_size, int rank_id,
                                      int64_t rows, int64_t h, mc2_dtype x_dtype, mc2_dtype scale_dtype,
                                      const void* out, mc2_dtype out_dtype) {
  mc2_status s = check_quant_reduce("quant_reduce_scatter", x, scales, world_size, rows, h, x_dtype, scale_dtype,
                                    out, out_dtype);
  if (s != MC2_OK) return s;
  if (rank_id < 0 || rank_id >= world_size) return fail(MC2_ERR_SHAPE, "quant_reduce_scatter: rank_id out of range");
  if (rows % world_size != 0)
    return fail(MC2_ERR_SHAPE, "quant_reduce_scatter: rows must be divisible by world_size");
  return MC2_OK;
}

}  // namespace mc2
