// K9: streaming read of the int8 GEMM's weight into the last-level cache
// (MALL) for the GEMM, in AlltoAllQuantMatmul (A16W8 and full quantisation).
//
// The GEMM reads B = x2 (r h, n) int8 step by step, 128 rows of K at a time,
// from 256 workgroups that drift apart over the K loop.  Fetched from HBM in
// that order it took 288-290 us per call in the benchmark step (350 us after
// a 1 GB write), and 193-210 us when x2 had just passed through the caches:
// its loads then return at last-level-cache latency, and the workgroups of an
// XCD stay close enough to share their L2 (fetched bytes: 890-990 MB against
// the 504 MB floor).  One linear pass over x2 (235 MB at the A16W8 shape)
// takes about 40 us; run on a side stream beside the GEMM (which leaves CU
// slots free: one 364-register wavefront per SIMD) it stays ahead of the
// GEMM's K loop and costs the call little.  The bytes are only loaded: each
// thread folds its loads into one word and stores it (to a library-owned
// array nothing reads) only if it equals a value passed at launch, so the
// loads cannot be dropped and next to nothing is written.
#include "device.hpp"
#include "kernels.hpp"

namespace mc2 {

// Where a thread would put its folded word: never read; written only when the
// word equals `magic` (a kernel argument, so the compiler has to load and
// fold).  External linkage, so the compiler cannot prove the store dead.
__device__ unsigned prefetch_sink[256];

namespace {

constexpr int kPrefetchThreads = 256;
constexpr int kPer = 8;  // 16-byte loads in flight per thread

__global__ __launch_bounds__(kPrefetchThreads) void prefetch_kernel(const u32x4* __restrict__ src, int64_t chunks,
                                                                    unsigned magic) {
  const int64_t c0 = (int64_t)blockIdx.x * (kPer * kPrefetchThreads) + threadIdx.x;
  u32x4 v[kPer];
#pragma unroll
  for (int j = 0; j < kPer; j++) {
    const int64_t c = c0 + (int64_t)j * kPrefetchThreads;
    v[j] = src[c < chunks ? c : chunks - 1];  // default policy: the lines are kept
  }
  unsigned x = 0;
#pragma unroll
  for (int j = 0; j < kPer; j++) x ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  if (x == magic) prefetch_sink[threadIdx.x] = x;
}

}  // namespace

hipError_t launch_prefetch(const void* p, int64_t bytes, hipStream_t s) {
  if (!p || bytes < 16 || reinterpret_cast<uintptr_t>(p) % 16 != 0) return hipSuccess;  // nothing worth reading
  const int64_t chunks = bytes / 16, per = (int64_t)kPer * kPrefetchThreads;
  const int64_t blocks = (chunks + per - 1) / per;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  prefetch_kernel<<<(unsigned)blocks, kPrefetchThreads, 0, s>>>(static_cast<const u32x4*>(p), chunks, 0x9E3779B9u);
  return hipGetLastError();
}

}  // namespace mc2
