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
  // arrival emulation (ready_flags NULL when unused): A is read from
  // gather_out; rows [g rows_chunk, (g+1) rows_chunk) x columns
  // [s slab_cols, (s+1) slab_cols) may be read once
  // ready_flags[g * slabs + s] == ready_value.  rows_chunk must be a
  // multiple of gemm16_tile_rows(m, n, b_kmajor) and slab_cols of 64.  Tile row
  // first_row_tile is handed out first; *status_flag counts wavefronts
  // whose wait timed out after wait_ticks ticks of the 100 MHz real-time
  // counter (they read A from a_parts instead).
  const unsigned* ready_flags;
  unsigned ready_value;
  uint64_t wait_ticks;
  int64_t rows_chunk;
  int64_t slab_cols;
  int slabs;
  int first_row_tile;
  unsigned* status_flag;
  // reduce-scatter epilogue (rs_out NULL when unused): rows [rs_row0,
  // rs_row0 + rs_rows) of C are not stored; rs_out row t = round(sum over
  // ranks j < rs_ranks in order of (j == rs_rank ? C row rs_row0 + t :
  // rs_recv[j] row t)), the sum in fp32.  rs_recv[j] and rs_out have n columns.
  void* rs_out;
  const void* rs_recv[kMaxRanks];
  int rs_ranks, rs_rank;
  int64_t rs_row0, rs_rows;
  // bias (n values of dtype, NULL: none) added before the output's rounding:
  // to every row of C, or with rs_out only to the reduced block (rs_out row t
  // = round(sum + bias)); the rows C sends to other ranks carry none.
  const void* bias;
};
hipError_t launch_gemm16(const GemmArgs& a, hipStream_t s);
// The fp16 part of launch_gemm16 (its own translation unit).
hipError_t launch_gemm16_f16(const GemmArgs& a, hipStream_t s);
// Tile height (rows of C per workgroup) launch_gemm16 uses for an (m, n) C
// with A K-major and B K-major (b_kmajor = 1) or N-major.
int gemm16_tile_rows(int64_t m, int64_t n, int b_kmajor);

// Default longest wait of the arrival GEMM for one piece: 200 ms of the
// 100 MHz real-time counter.
constexpr uint64_t kArrivalWaitTicks = 20000000ull;

// ---- grad_bias: gb[j] = round(sum over rows i of dy[i][j]), (m, n) 16-bit dy,
// the sum in fp64, rounded once to the same 16-bit type
hipError_t launch_bias_grad(const void* dy, int64_t m, int64_t n, int dtype, void* gb, hipStream_t s);

// ---- arrival emulation: copy of the shards into gather_out piece by piece
// (row chunk g, slab s of K), each piece followed by its ready flag
// (flags[g * slabs + s] = epoch; only for slabs s < raised_slabs, which is
// `slabs` except under the time-out test hook).  Row chunk g covers gathered rows
// [g rows_chunk, (g+1) rows_chunk); one workgroup per piece, slab by slab,
// row chunk first_chunk first within a slab.
struct ArrivalArgs {
  const void* shards[kMaxRanks];
  void* gather_out;
  unsigned* flags;
  int64_t block_rows;  // rows per shard
  int64_t k;           // elements per row (16-bit elements)
  int64_t rows_chunk;
  int64_t slab_cols;
  int slabs;
  int raised_slabs;    // slabs whose flags are raised (the others' pieces are copied only)
  int chunks;          // row chunks in the gathered matrix
  int r, first_chunk;
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
  // A (m, k): element (row, kk) at a + (kk / kseg) kseg_stride + row a_ld + kk % kseg
  // (kseg = 0: a plain row-major (m, k) matrix)
  const int8_t* a;
  int64_t a_ld, kseg, kseg_stride, a_bytes;
  void* permuted_out;    // optional (m, k) copy of A as the GEMM reads it
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

// ---- K7: int4 codes (two per byte, low nibble first) widened to int8
struct WidenArgs {
  const uint8_t* src[2];  // packed codes, 16-byte aligned (a range of 0 bytes: unused)
  int8_t* dst[2];         // 2 bytes[i] int8 values, 16-byte aligned
  int64_t bytes[2];       // packed bytes of each range
  int64_t blocks0;        // set by the launcher
};
hipError_t launch_widen_int4(const WidenArgs& a, hipStream_t s);

// ---- K9: one streaming read of `bytes` at p (16-byte aligned) into the caches (no writes)
hipError_t launch_prefetch(const void* p, int64_t bytes, hipStream_t s);

}  // namespace mc2
