/*
 * mc2.h -- C ABI of libmc2: the per-rank compute of the MC2 fused
 * communication + matmul operators on one AMD Instinct MI355X (gfx950).
 *
 * On one GPU the r ranks' shards are r separate device buffers, so the
 * collective steps of each operator (AllGather, AlltoAll) become the gather
 * and permute addressing the kernels do as they read.  No call here talks to
 * another GPU.
 *
 * Conventions for every entry point
 *  - Tensors are caller-owned DEVICE pointers (hipMalloc or torch storage),
 *    row-major and contiguous unless a layout flag says otherwise.  Arrays of
 *    pointers ("shards", "x", "scales") are HOST arrays of device pointers.
 *    Every tensor pointer must be 16-byte aligned.
 *  - `stream` is a hipStream_t passed as void*; NULL means the default
 *    stream.  Work is enqueued asynchronously on it; the call returns once
 *    the work is enqueued.
 *  - Arguments are validated on the host before anything is enqueued.  On a
 *    validation error nothing is written and no device call is made.
 *  - Every call returns an mc2_status.  MC2_ERR_HIP means a HIP runtime call
 *    failed; mc2_last_error() then gives the text (per thread).  Nothing
 *    aborts and no C++ exception crosses this interface.
 *  - The library allocates no caller-visible memory and frees none.  Results
 *    are deterministic: the same inputs give the same bits on every run.
 *  - Calls on different streams may run concurrently, except that
 *    MC2_AG_ARRIVAL calls on one device must not overlap each other.
 */
#ifndef MC2_H_
#define MC2_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MC2_OK = 0,
  MC2_ERR_NULL = 1,        /* a required pointer is NULL */
  MC2_ERR_SHAPE = 2,       /* a size breaks the operator's constraints */
  MC2_ERR_DTYPE = 3,       /* dtype, or dtype combination, not supported */
  MC2_ERR_UNSUPPORTED = 4, /* allowed by the operator but not provided here */
  MC2_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required */
  MC2_ERR_NO_DEVICE = 6,   /* no HIP device, or the current device is not gfx950 */
  MC2_ERR_HIP = 7,         /* a HIP runtime call failed (see mc2_last_error) */
  MC2_ERR_ALIGN = 8        /* a tensor pointer is not 16-byte aligned */
} mc2_status;

typedef enum {
  MC2_F32 = 0,
  MC2_F16 = 1,
  MC2_BF16 = 2,
  MC2_I8 = 3,
  MC2_I32 = 4,
  MC2_F8E4M3FN = 5, /* OCP FLOAT8_E4M3FN: bias 7, max 448, no infinities */
  MC2_F8E5M2 = 6,   /* OCP FLOAT8_E5M2: bias 15, IEEE-style inf / NaN */
  MC2_E8M0 = 7      /* OCP MX scale: unsigned exponent, value 2^(b - 127), 0xFF NaN */
} mc2_dtype;

/* Quant modes of the AlltoAllQuantMatmul page (x1QuantMode / x2QuantMode). */
typedef enum {
  MC2_QUANT_NONE = 0,
  MC2_QUANT_PERTENSOR = 1,
  MC2_QUANT_PERCHANNEL = 2,
  MC2_QUANT_PERTOKEN = 3,
  MC2_QUANT_PERGROUP = 4,
  MC2_QUANT_PERBLOCK = 5,
  MC2_QUANT_MX = 6,
  MC2_QUANT_PERTOKEN_DYNAMIC = 7
} mc2_quant_mode;

typedef enum {
  /* the GEMM reads each rank's rows straight from its shard and the
     workgroups of the first column tile also write gather_out */
  MC2_AG_FUSED_WRITE = 0,
  /* arrival emulation: on a side stream a copy kernel fills gather_out
     piece by piece -- row chunks of the GEMM's tile height times up to 16
     slabs of K, the local rank's (rank_id) rows first -- raising a ready
     flag per piece; the GEMM reads A from gather_out and issues the loads
     of each slab of K only once its piece has arrived, so compute starts on
     the first slab while later ones are still being copied.  The side
     stream is forked from and joined back into `stream`.  A wavefront that
     waits longer than 200 ms for a piece reads the rest of its rows from
     the shards instead (the result is the same) and is counted by
     mc2_allgather_arrival_fallbacks. */
  MC2_AG_ARRIVAL = 1
} mc2_ag_mode;

/*
 * AllGatherMatmul -- torch_npu.npu_all_gather_base_mm (Ascend PyTorch API
 * page, "function", "outputs" and "constraints" sections):
 *   gather_out = AllGather_m(shards)           rows [i m_local, (i+1) m_local) = shard i
 *   out        = gather_out @ x2               fp32 accumulation, rounded to `dtype`
 *
 * shards      host array of world_size device pointers, each (m_local, k) of `dtype`
 * world_size  2, 4 or 8
 * k           contraction size, 256 <= k < 65535
 * x2          (k, n) row-major if x2_trans == 0; if x2_trans == 1 the buffer
 *             holds x2^T as (n, k) row-major (a transposed view, which the
 *             op accepts for x2 but not for the input)
 * dtype       MC2_F16 or MC2_BF16, the type of shards, x2, out, gather_out
 * out         (world_size m_local, n)
 * gather_out  (world_size m_local, k), or NULL when the gathered input is not
 *             wanted (the op's gather_output = false); MC2_AG_ARRIVAL needs it
 * mode        MC2_AG_FUSED_WRITE or MC2_AG_ARRIVAL
 * rank_id     the calling rank, 0 <= rank_id < world_size: its block is
 *             local and is consumed first in MC2_AG_ARRIVAL mode (unused in
 *             MC2_AG_FUSED_WRITE mode)
 * The op's bias is not accepted (the page allows only a zero bias), and
 * gather_index / comm_turn exist only with their default 0, so they are not
 * arguments.
 */
mc2_status mc2_allgather_matmul(const void* const* shards, int world_size, int64_t m_local,
                                int64_t k, const void* x2, int64_t n, int x2_trans,
                                mc2_dtype dtype, void* out, void* gather_out, mc2_ag_mode mode,
                                int rank_id, void* stream);

/*
 * The column-parallel layer's forward with its bias -- hyper_parallel mc2.py,
 * AllGatherMatmulFunction.forward: the fused op runs without a bias and the
 * layer then adds it, out = AllGather_m(shards) @ x2 + bias.  Same arguments
 * and errors as mc2_allgather_matmul plus
 * bias        (n) of `dtype`, required (16-byte aligned)
 * The bias is added to the fp32 accumulator before the single rounding of
 * out (the listing rounds the product to `dtype` and then adds; the two
 * differ by at most one rounding of the output).  gather_out is unchanged.
 */
mc2_status mc2_allgather_matmul_bias(const void* const* shards, int world_size, int64_t m_local, int64_t k,
                                     const void* x2, int64_t n, int x2_trans, mc2_dtype dtype, const void* bias,
                                     void* out, void* gather_out, mc2_ag_mode mode, int rank_id, void* stream);

/*
 * Number of GEMM wavefronts of MC2_AG_ARRIVAL calls on the current device
 * whose wait for a piece of gather_out timed out since the last reset (each
 * read its rows from the shards instead, so results are unaffected).
 * Waits for the device to be idle; reset != 0 clears the count afterwards.
 * A nonzero count means the copies did not feed the GEMM in time, so that
 * call did not pipeline copies with compute.
 */
mc2_status mc2_allgather_arrival_fallbacks(int reset, unsigned* count);

/*
 * Column-parallel backward, local share of dX -- hyper_parallel mc2.py,
 * AllGatherMatmulFunction.backward: dX = ReduceScatter_m(dY @ W).  This call
 * computes one rank's dY @ W before the reduce-scatter:
 *   dx_partial (m, k) = dy (m, n_local) @ w (n_local, k)
 * w is the nn.Linear weight in its (out, in) = (n_local, k) layout.  The
 * contraction runs over n_local, which the fused kernel requires to lie in
 * [256, 65535).  fp32 accumulation, output rounded to `dtype` (F16 / BF16).
 */
mc2_status mc2_matmul_grad_input(const void* dy, const void* w, int64_t m, int64_t n_local,
                                 int64_t k, mc2_dtype dtype, void* dx_partial, void* stream);

/*
 * MatmulReduceScatter, the share of rank rank_id of world_size --
 * hyper_parallel mc2.py, module docstring and MatmulReduceScatterFunction:
 * the row-parallel forward Y = ReduceScatter_m(X @ W^T) (x2 = W^T, pass W
 * with x2_trans = 1), and AllGatherMatmulFunction.backward's
 * dX = ReduceScatter_m(dY @ W) (x2 = W, x2_trans = 0).  This rank computes
 * its partial x @ x2 and reduces its own row block with the blocks the other
 * ranks send it:
 *   partial_out (m, n) = round(x (m, k) @ x2), fp32 accumulation; the rows
 *       of other ranks' blocks are written (they are what this rank sends),
 *       the rows [rank_id m/ws, (rank_id+1) m/ws) of its own block are not;
 *   out (m / ws, n) = round(B_0 + B_1 + ... + B_{ws-1}), summed in fp32 in
 *       rank order, B_j = recv[j] for j != rank_id and the rounded own-block
 *       rows of x @ x2 for j == rank_id.
 * Reading of the pages: each rank's partial is a matmul output, so it is
 * rounded to `dtype` before the reduction; the pages fix no order or
 * precision for the sum, so it runs in fp32 in rank order and is rounded
 * once.  The tiles of the own block run last, so on several GPUs the
 * received blocks have the whole GEMM to arrive; the sum is a second pass
 * on `stream` after the GEMM, in place in `out`.
 *
 * x         (m, k) row-major; k is the contraction size of the fused kernel,
 *           in [256, 65535); m divisible by world_size
 * x2        (k, n) row-major, or with x2_trans (n, k) row-major
 * recv      world_size pointers: recv[j], j != rank_id, is a (m / ws, n)
 *           row-major block of `dtype`; recv[rank_id] is not read (may be NULL)
 * out, partial_out  as above, of `dtype` (F16 or BF16)
 * All pointers are caller-owned device memory, 16-byte aligned; out must not
 * overlap partial_out or a received block (the sum is formed in place in out).
 */
mc2_status mc2_matmul_reduce_scatter(const void* x, const void* x2, int world_size, int rank_id, int64_t m,
                                     int64_t k, int64_t n, int x2_trans, mc2_dtype dtype, const void* const* recv,
                                     void* out, void* partial_out, void* stream);

/*
 * The row-parallel layer's forward with its bias -- hyper_parallel mc2.py,
 * MatmulReduceScatterFunction.forward: out = ReduceScatter_m(x @ x2) + bias.
 * Same arguments and errors as mc2_matmul_reduce_scatter plus
 * bias        (n) of `dtype`, required (16-byte aligned)
 * The bias enters only the reduced block: out = round(B_0 + ... + B_{ws-1}
 * + bias), summed in fp32 in rank order then the bias, rounded once;
 * partial_out (what this rank sends) carries no bias.
 */
mc2_status mc2_matmul_reduce_scatter_bias(const void* x, const void* x2, int world_size, int rank_id, int64_t m,
                                          int64_t k, int64_t n, int x2_trans, mc2_dtype dtype,
                                          const void* const* recv, const void* bias, void* out, void* partial_out,
                                          void* stream);

/*
 * Bias gradient of the tensor-parallel linear layer -- hyper_parallel mc2.py,
 * AllGatherMatmulFunction.backward (grad_bias = grad_out.sum(dim=0)) and
 * MatmulReduceScatterFunction.backward (the same over the gathered
 * grad_out_full, i.e. gather_out of the backward's AllGatherMatmul):
 *   grad_bias[j] = round( sum over i < m of dy[i][j] )
 * dy (m, n) row-major of `dtype` (F16 / BF16), grad_bias (n) of `dtype`.
 * The sum runs in fp64 and is rounded once: exact, hence independent of the
 * summation order, whenever a column's values span fewer than about
 * 53 - 11 - log2(m) binades.
 */
mc2_status mc2_bias_grad(const void* dy, int64_t m, int64_t n, mc2_dtype dtype, void* grad_bias, void* stream);

/*
 * Column-parallel backward, weight gradient -- hyper_parallel mc2.py,
 * AllGatherMatmulFunction.backward: dW = dY^T @ AllGather_m(X), where
 * AllGather_m(X) is the gather_out saved by the forward.
 *   dw (n_local, k) = dy (m, n_local)^T @ ag_x (m, k)
 * fp32 accumulation, output rounded to `dtype` (F16 / BF16).
 */
mc2_status mc2_matmul_grad_weight(const void* dy, const void* ag_x, int64_t m, int64_t n_local,
                                  int64_t k, mc2_dtype dtype, void* dw, void* stream);

/*
 * Workspace bytes mc2_alltoall_quant_matmul needs for these sizes (stage one
 * of the two-stage call of the aclnnAlltoAllQuantMatmul page, "prototype").
 */
mc2_status mc2_alltoall_quant_matmul_workspace_size(int rank_size, int64_t bs, int64_t h,
                                                    int64_t n, size_t* bytes);

/*
 * AlltoAllQuantMatmul, A16W8 with dynamic per-token quantisation (x1 mode 7,
 * x2 mode 2) -- aclnnAlltoAllQuantMatmul page, "function" formulas:
 *   commOut      = AlltoAll(x1.view(rank_size, bs / rank_size, h))
 *   P            = commOut.permute(1, 0, 2).view(bs / rank_size, rank_size h)
 *   q, x1_scale  = Quant(P * x1_smooth)       per token: scale = absmax / 127,
 *                                              q = clamp(rint(y / scale), -127, 127)
 *   acc          = q @ x2                      exact int32
 *   out          = acc * x1_scale * x2_scale + bias
 * On one GPU x1 is this rank's buffer after the AlltoAll: block j of
 * x1.view(rank_size, bs / rank_size, h) is what rank j sent.
 *
 * x1          (bs, h) of x1_dtype (MC2_BF16 or MC2_F16)
 * rank_size   2, 4 or 8; bs divisible by rank_size; bs, n <= INT32_MAX;
 *             rank_size h divisible by 16 and in [1, 35000] (A16W8)
 * x2          (rank_size h, n) int8, row-major, contiguous
 * x2_scale    (n) fp32 per-channel scale
 * x1_smooth   (rank_size h) of x1_dtype, or NULL for no smoothing
 * bias        (n) of x1_dtype, or NULL for a zero bias
 * out         (bs / rank_size, n) of x1_dtype
 * permuted_out, q_out, x1_scale_out, acc_out: optional (NULL) copies of P
 *             (x1_dtype), q (int8), x1_scale (fp32) and acc (int32)
 * workspace   device memory of at least the size the sizing call returns
 */
mc2_status mc2_alltoall_quant_matmul(const void* x1, int rank_size, int64_t bs, int64_t h,
                                     mc2_dtype x1_dtype, const int8_t* x2, int64_t n,
                                     const float* x2_scale, const void* x1_smooth,
                                     const void* bias, void* out, void* permuted_out,
                                     int8_t* q_out, float* x1_scale_out, int32_t* acc_out,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * mc2_alltoall_quant_matmul without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and errors as
 * mc2_alltoall_quant_matmul, minus workspace and workspace_bytes: the
 * workspace is a device array inside the library, MC2_NOALLOC_SCRATCH_BYTES
 * (48 MiB) per GPU, held from the library's first use on that GPU until the
 * process ends.  Sizes whose workspace (mc2_alltoall_quant_matmul_workspace_size)
 * exceeds it are rejected with MC2_ERR_WORKSPACE before any device call; at
 * rank_size h = 32768 that allows bs / rank_size up to 1535 tokens.  This call
 * allocates nothing.  Every call on a GPU shares that GPU's array, so calls
 * that overlap in time on one GPU (other streams, other host threads) race
 * on it and must be serialised by the caller; the array keeps the last
 * call's contents, which the next call overwrites before reading.
 */
#define MC2_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)
mc2_status mc2_alltoall_quant_matmul_noalloc(const void* x1, int rank_size, int64_t bs, int64_t h,
                                             mc2_dtype x1_dtype, const int8_t* x2, int64_t n,
                                             const float* x2_scale, const void* x1_smooth,
                                             const void* bias, void* out, void* permuted_out,
                                             int8_t* q_out, float* x1_scale_out, int32_t* acc_out,
                                             void* stream);

/*
 * AlltoAllQuantMatmul, full quantisation (x1 mode 3, per-token; x2 mode 2,
 * per-channel) -- aclnnAlltoAllQuantMatmul page, "function" formulas, the
 * full-quant case: x1 arrives already int8, with one scale per token.
 *   P      = AlltoAll(x1.view(rank_size, bs / rank_size, h)).permute(1, 0, 2)
 *            .view(bs / rank_size, rank_size h)           (int8 bytes)
 *   acc    = P @ x2                                        exact int32
 *   out    = acc * x1_scale * x2_scale + bias              fp32, rounded once
 * The page prints the product as "x1 @ x2"; it is read as P @ x2 (the
 * permute is defined just before it and only P has matching shapes).
 * x1_scale holds one fp32 scale per token of P.  The permute is the GEMM's
 * load addressing: nothing is materialised and no workspace is needed.
 *
 * x1          (bs, h) int8; sizes as for mc2_alltoall_quant_matmul
 * x1_scale    (bs / rank_size) fp32
 * x2          (rank_size h, n) int8, row-major, contiguous
 * x2_scale    (n) fp32 per-channel scale
 * bias        (n) of out_dtype, or NULL for a zero bias
 * out         (bs / rank_size, n) of out_dtype (MC2_BF16 or MC2_F16)
 * permuted_out, acc_out: optional (NULL) copies of P (int8) and acc (int32)
 */
mc2_status mc2_alltoall_quant_matmul_static(const int8_t* x1, int rank_size, int64_t bs, int64_t h,
                                            const float* x1_scale, const int8_t* x2, int64_t n,
                                            const float* x2_scale, const void* bias, void* out,
                                            mc2_dtype out_dtype, int8_t* permuted_out, int32_t* acc_out,
                                            void* stream);

/*
 * Reading of the int4 formats of A16W4 / A4W4 (aclnnAlltoAllQuantMatmul page,
 * "constraints": A16W4 needs N even, A4W4 needs H and N even; the quantised
 * x1 dtype is INT8 only): two's-complement int4 codes (-8..7), two per byte
 * along the last dimension, value 2i in the low nibble of byte i and value
 * 2i + 1 in the high nibble.  The library widens int4 operands to int8 in the
 * workspace (exactly) before the int8 GEMM.
 *
 * AlltoAllQuantMatmul A16W4: mc2_alltoall_quant_matmul's dynamic per-token
 * chain (x1 quantised to int8 per token) with an int4 weight:
 * x2 (rank_size h, n / 2) bytes of int4 codes; n must be even.  Every other
 * argument and the results are those of mc2_alltoall_quant_matmul; acc is
 * exact int32.  The workspace (16-byte aligned) holds
 * mc2_alltoall_quant_matmul_a16w4_workspace_size bytes: the A16W8 workspace
 * plus rank_size h n bytes for the widened weight.
 */
mc2_status mc2_alltoall_quant_matmul_a16w4_workspace_size(int rank_size, int64_t bs, int64_t h, int64_t n,
                                                          size_t* bytes);
mc2_status mc2_alltoall_quant_matmul_a16w4(const void* x1, int rank_size, int64_t bs, int64_t h,
                                           mc2_dtype x1_dtype, const uint8_t* x2, int64_t n, const float* x2_scale,
                                           const void* x1_smooth, const void* bias, void* out, void* permuted_out,
                                           int8_t* q_out, float* x1_scale_out, int32_t* acc_out, void* workspace,
                                           size_t workspace_bytes, void* stream);

/*
 * AlltoAllQuantMatmul A4W4 (full quantisation, x1 mode 3, x2 mode 2): the
 * chain of mc2_alltoall_quant_matmul_static with int4 activations and weight.
 *   P    = AlltoAll(x1.view(rank_size, bs / rank_size, h)).permute(1, 0, 2)
 *          .view(bs / rank_size, rank_size h)        (int4 codes)
 *   acc  = P @ x2                                     exact int32
 *   out  = acc * x1_scale * x2_scale + bias           fp32, rounded once
 * x1        (bs, h / 2) bytes of int4 codes; h even; rank_size h in [1, 35000]
 * x1_scale  (bs / rank_size) fp32, one per token of P
 * x2        (rank_size h, n / 2) bytes of int4 codes; n even
 * x2_scale  (n) fp32; bias (n) of out_dtype or NULL; out (bs / rank_size, n)
 * acc_out   optional (bs / rank_size, n) int32
 * workspace 16-byte aligned, mc2_alltoall_quant_matmul_a4w4_workspace_size
 *           bytes (bs h + rank_size h n, rounded up): both operands widened
 *           to int8.  The permute is the GEMM's load addressing.
 */
mc2_status mc2_alltoall_quant_matmul_a4w4_workspace_size(int rank_size, int64_t bs, int64_t h, int64_t n,
                                                         size_t* bytes);
mc2_status mc2_alltoall_quant_matmul_a4w4(const uint8_t* x1, int rank_size, int64_t bs, int64_t h,
                                          const float* x1_scale, const uint8_t* x2, int64_t n,
                                          const float* x2_scale, const void* bias, void* out, mc2_dtype out_dtype,
                                          int32_t* acc_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * QuantAllReduce -- QuantAllReduce README ("function" formula, parameter
 * table, constraints):
 *   out = sum over ranks i of dequant(x[i])   with dequant = x * its scale
 * The sum is exact in fp64, in rank order, and rounded once to out_dtype.
 *
 * x           host array of world_size device pointers, each (rows, h) of
 *             x_dtype; rows = b s for a (b, s, h) tensor
 * scales      host array of world_size device pointers:
 *             scale_dtype MC2_F32 : (rows, h / 128) fp32, one scale per token
 *                                   and 128-element group (pertoken-pergroup)
 *             scale_dtype MC2_E8M0: (rows, h / 64, 2) E8M0, i.e. one scale per
 *                                   32-element block (mx)
 * x_dtype     with MC2_F32 scales: MC2_I8, MC2_F8E4M3FN or MC2_F8E5M2;
 *             with MC2_E8M0 scales: MC2_F8E4M3FN or MC2_F8E5M2
 * world_size  2, 4 or 8;  h in [1024, 8192] and a multiple of 128
 * out         (rows, h) of out_dtype: MC2_F32, MC2_F16 or MC2_BF16
 */
mc2_status mc2_quant_all_reduce(const void* const* x, const void* const* scales, int world_size,
                                int64_t rows, int64_t h, mc2_dtype x_dtype,
                                mc2_dtype scale_dtype, void* out, mc2_dtype out_dtype,
                                void* stream);

/*
 * QuantReduceScatter, the share of rank rank_id -- named beside
 * QuantAllReduce in the QuantAllReduce README's constraints (the two may run
 * back to back in one communication domain); read as the reduce-scatter
 * form of the same formula: this rank keeps rows [rank_id rows/ws,
 * (rank_id+1) rows/ws) of output = Reduce(AllGather(scales) *
 * AllGather(x)), summed over ranks in order exactly as mc2_quant_all_reduce.
 * Arguments as for mc2_quant_all_reduce; rows must be divisible by
 * world_size and out is (rows / world_size, h) of out_dtype.
 */
mc2_status mc2_quant_reduce_scatter(const void* const* x, const void* const* scales, int world_size, int rank_id,
                                    int64_t rows, int64_t h, mc2_dtype x_dtype, mc2_dtype scale_dtype, void* out,
                                    mc2_dtype out_dtype, void* stream);

/* Static text for a status code. */
const char* mc2_status_string(mc2_status s);

/* Text of the last error on this thread ("" if none). */
const char* mc2_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MC2_H_ */
