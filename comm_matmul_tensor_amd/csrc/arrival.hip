// Arrival emulation for AllGatherMatmul (torch_npu npu_all_gather_base_mm
// page, "function": communication and matmul run as a pipeline).
//
// On one GPU the peers' shards are already in HBM, so their "arrival" is
// modelled by a copy kernel on a side stream: shard i is copied into row
// block i of gather_out in chunks of rows, and each chunk raises its own
// ready flag once its bytes are visible to every XCD.  The GEMM's workgroups
// poll the flags of the chunks their tile covers (gemm_mfma.hpp), so tiles
// start as their rows land.  Workgroups are handed out local block first,
// then the other blocks in rank order after it, as a ring AllGather delivers
// them.
#include "device.hpp"
#include "kernels.hpp"

namespace mc2 {
namespace {

constexpr int kCopyThreads = 256;

__global__ __launch_bounds__(kCopyThreads) void arrive_kernel(ArrivalArgs a) {
  const int w = blockIdx.x;
  const int blk = (a.first + w / a.chunks) % a.r, c = w % a.chunks;
  const int64_t row0 = (int64_t)c * a.chunk_rows;
  const int64_t rows = (row0 + a.chunk_rows <= a.block_rows ? a.chunk_rows : a.block_rows - row0);
  const int64_t bytes = rows * a.row_bytes;
  const uint8_t* src = static_cast<const uint8_t*>(a.shards[blk]) + row0 * a.row_bytes;
  uint8_t* dst = static_cast<uint8_t*>(a.gather_out) + ((int64_t)blk * a.block_rows + row0) * a.row_bytes;
  if (bytes > 0) {
    if ((((uintptr_t)src | (uintptr_t)dst | (uintptr_t)bytes) & 15) == 0) {
      const u32x4* s = reinterpret_cast<const u32x4*>(src);
      u32x4* d = reinterpret_cast<u32x4*>(dst);
      const int64_t n = bytes / 16;
      int64_t i = threadIdx.x;
      for (; i + 3 * kCopyThreads < n; i += 4 * kCopyThreads) {
        const u32x4 v0 = s[i], v1 = s[i + kCopyThreads], v2 = s[i + 2 * kCopyThreads], v3 = s[i + 3 * kCopyThreads];
        d[i] = v0;
        d[i + kCopyThreads] = v1;
        d[i + 2 * kCopyThreads] = v2;
        d[i + 3 * kCopyThreads] = v3;
      }
      for (; i < n; i += kCopyThreads) d[i] = s[i];
    } else {  // 16-bit elements, any row length
      const uint16_t* s = reinterpret_cast<const uint16_t*>(src);
      uint16_t* d = reinterpret_cast<uint16_t*>(dst);
      for (int64_t i = threadIdx.x; i < bytes / 2; i += kCopyThreads) d[i] = s[i];
    }
  }
  // Every wave makes its stores visible device-wide (the XCDs' L2s are not
  // coherent with each other), then one thread raises the chunk's flag.
  __atomic_thread_fence(__ATOMIC_RELEASE);
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_store(a.flags + (int64_t)blk * a.chunks + c, a.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

}  // namespace

hipError_t launch_arrival_copy(const ArrivalArgs& a, hipStream_t s) {
  if (a.r < 1 || a.r > kMaxRanks || a.chunks < 1 || a.chunk_rows < 1 || a.block_rows < 1 || a.row_bytes < 2 ||
      (int64_t)a.chunks * a.chunk_rows < a.block_rows || a.first < 0 || a.first >= a.r)
    return hipErrorInvalidValue;
  arrive_kernel<<<a.r * a.chunks, kCopyThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mc2
