// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace mc2 {

constexpr int kMaxRanks = 8;

// ---- K4: QuantAllReduce dequant-sum
struct QarArgs {
  const void* x[kMaxRanks];
  const void* scales[kMaxRanks];
  void* out;
  int64_t total;  // rows * h
  int64_t h;
  int r;
  int x_dtype, scale_dtype, out_dtype;  // DT_* codes
};
hipError_t launch_dequant_sum(const QarArgs& a, hipStream_t s);

// ---- K1: 16-bit float GEMM  C (m, n) = A (m, k) @ B (k, n), fp32 accumulation
// A is either gathered from `a_parts` row blocks (each (rows_per_part, k),
// K-contiguous) or a single matrix (a_parts = 1).  a_kmajor = 0 means A is
// stored transposed, (k, m) row-major.  b_kmajor = 1 means B is stored as
// (n, k) row-major; 0 means (k, n) row-major.
struct GemmArgs {
  const void* a_parts[kMaxRanks];
  int num_parts;
  int64_t rows_per_part;
  int a_kmajor;
  const void* b;
  int b_kmajor;
  void* c;
  void* gather_out;  // optional copy of the gathered A (only with a_kmajor)
  int64_t m, n, k;
  int dtype;  // DT_F16 or DT_BF16
  int tile_order_cols;  // set by the launcher: XCD tile order walks columns of tiles
  // arrival emulation (ready_flags NULL when unused): rows of part i of A
  // are read from gather_out once the flags of their chunks equal
  // ready_value (flag i * chunks + c covers rows [c chunk_rows, (c+1)
  // chunk_rows) of part i); the tiles of part first_part come first;
  // *status_flag counts workgroups whose wait timed out (they read the part
  // from a_parts instead)
  const unsigned* ready_flags;
  unsigned ready_value;
  int first_part;
  int chunks;
  int64_t chunk_rows;
  unsigned* status_flag;
};
hipError_t launch_gemm16(const GemmArgs& a, hipStream_t s);

// ---- arrival emulation: copy of the shards into gather_out, chunk by chunk,
// each chunk followed by its ready flag (flags[b * chunks + c] = epoch)
struct ArrivalArgs {
  const void* shards[kMaxRanks];
  void* gather_out;
  unsigned* flags;
  int64_t block_rows;  // rows per shard
  int64_t row_bytes;   // bytes per row
  int64_t chunk_rows;  // rows per chunk
  int chunks;          // chunks per shard
  int r, first;        // shard count; the block copied first
  unsigned epoch;
};
hipError_t launch_arrival_copy(const ArrivalArgs& a, hipStream_t s);

// ---- K2: permute + smooth + per-token dynamic int8 quantisation
struct QuantArgs {
  const void* x1;       // (bs, h), 16-bit
  const void* smooth;   // (r h) or NULL
  int8_t* q;            // (bs / r, r h)
  float* s1;            // (bs / r)
  void* permuted;       // optional (bs / r, r h) copy of the permuted input
  int64_t bs, h;
  int r;
  int dtype;
};
hipError_t launch_permute_quant(const QuantArgs& a, hipStream_t s);

// ---- K3: int8 GEMM with the fused dequant epilogue
struct GemmI8Args {
  const int8_t* a;       // (m, k) row-major
  const int8_t* b;       // (k, n) row-major
  const float* s1;       // (m)
  const float* s2;       // (n)
  const void* bias;      // (n) 16-bit or NULL
  void* out;             // (m, n) 16-bit
  int32_t* acc_out;      // optional (m, n) raw accumulators
  int32_t* partials;     // split-K workspace
  unsigned* counters;    // split-K tile counters
  int64_t m, n, k;
  int dtype;
  int split_k;
};
size_t gemm_i8_workspace_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_i8(const GemmI8Args& a, hipStream_t s);

}  // namespace mc2
