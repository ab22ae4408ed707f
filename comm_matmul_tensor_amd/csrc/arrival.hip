// Arrival emulation for AllGatherMatmul (torch_npu npu_all_gather_base_mm
// page, "function": communication and matmul run as a pipeline).
//
// On one GPU the peers' shards are already in HBM, so their "arrival" is
// modelled by a copy kernel on a side stream that fills gather_out piece by
// piece: the gathered rows are cut into row chunks (a multiple of the GEMM's
// tile height) and K into slabs.  One workgroup copies one piece (row chunk
// g, slab s) and then raises that piece's flag.  Workgroups are handed out
// slab by slab, and within a slab from the local rank's rows on (as a ring
// AllGather delivers them), so the GEMM's tiles can start on the first slab
// of K while later slabs are still being copied.
//
// Visibility across XCDs: the copy's stores carry the device-scope cache
// policy (sc1), so they write through the XCD's L2; once they have completed
// the piece is visible device-wide and its flag can be raised without any
// L2 write-back (see the end of copy_piece).  They are 16-byte buffer
// stores, whole 128-byte lines per eight lanes; 8-byte device-scope atomic
// stores (the same policy) serve a gather_out of 2 GiB or more and rows that
// are not whole 16-byte pieces.
#include <type_traits>

#include "device.hpp"
#include "kernels.hpp"

namespace mc2 {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kBatch = 16;  // 16-byte loads in flight per thread
constexpr int kPolicyDevice = 16;  // buffer store cache policy: sc1, coherent device-wide

// Copies piece w (slab w / chunks of row chunk (first_chunk + w % chunks) %
// chunks) and raises its flag.
__device__ __forceinline__ void copy_piece(const ArrivalArgs& a, const int w) {
  const int sl = w / a.chunks, g = (a.first_chunk + w % a.chunks) % a.chunks;
  const int64_t m = (int64_t)a.r * a.block_rows;
  const int64_t row0 = (int64_t)g * a.rows_chunk;
  const int64_t rows = row0 + a.rows_chunk <= m ? a.rows_chunk : m - row0;
  const int64_t c0 = (int64_t)sl * a.slab_cols;
  const int64_t cols = c0 + a.slab_cols <= a.k ? a.slab_cols : a.k - c0;
  uint16_t* gout = static_cast<uint16_t*>(a.gather_out);
  // one shard holds the whole chunk unless the chunk straddles a shard edge
  const int64_t b0 = row0 / a.block_rows;
  const bool one_shard = (row0 + rows - 1) / a.block_rows == b0;
  if ((a.k % 8 == 0) && (a.slab_cols % 8 == 0)) {
    // 16-byte pieces in row-major order; thread t takes pieces t, t + 256, ...
    // and steps its (row, piece) position without dividing.  kBatch loads per
    // thread are issued before their stores.  A chunk inside one shard (the
    // usual case) reads through that shard's pointer, loaded once for the
    // workgroup; a chunk across a shard edge finds each row's shard per lane.
    const int per_row = (int)(cols / 8), n = (int)rows * per_row;
    const bool buf = m * a.k * 2 < ((int64_t)1 << 31);  // byte offsets fit the buffer's 32 bits
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(gout, 0, buf ? (int)(m * a.k * 2) : 0, 0x00020000);
    const int dq = kCopyThreads / per_row, dc = kCopyThreads % per_row;
    const uint16_t* one_src = static_cast<const uint16_t*>(a.shards[b0]);
    const int64_t one_row0 = b0 * a.block_rows;
    // Straight-line batches: a lane whose j-th piece lies past the end
    // repeats its first piece (always valid: i0 < n), loading and storing the
    // same bytes to the same place again, so neither loads nor stores sit
    // behind per-lane branches (which made the compiler wait for every
    // earlier store before each store).
    auto copy = [&](auto ONE_, auto BUF_) {
      constexpr bool ONE = decltype(ONE_)::value, BUF = decltype(BUF_)::value;
      int r = (int)threadIdx.x / per_row, c = (int)threadIdx.x % per_row;
      for (int i0 = (int)threadIdx.x; i0 < n; i0 += kBatch * kCopyThreads) {
        u32x4 v[kBatch];
        int64_t dst[kBatch];
        int64_t R0 = 0, col0 = 0;
#pragma unroll
        for (int j = 0; j < kBatch; j++) {
          int64_t R = row0 + r, col = c0 + (int64_t)c * 8;
          if (j == 0) {
            R0 = R;
            col0 = col;
          } else if (i0 + j * kCopyThreads >= n) {
            R = R0;
            col = col0;
          }
          const uint16_t* src;
          if constexpr (ONE) {
            src = one_src + (R - one_row0) * a.k + col;
          } else {
            const int64_t bb = (int64_t)((uint32_t)R / (uint32_t)a.block_rows);
            src = static_cast<const uint16_t*>(a.shards[bb]) + (R - bb * a.block_rows) * a.k + col;
          }
          v[j] = *reinterpret_cast<const u32x4*>(src);
          dst[j] = R * a.k + col;
          r += dq;
          c += dc;
          if (c >= per_row) {
            c -= per_row;
            r += 1;
          }
        }
#pragma unroll
        for (int j = 0; j < kBatch; j++) {
          if constexpr (BUF) {
            __builtin_amdgcn_raw_buffer_store_b128(v[j], rsrc, (int)(dst[j] * 2), 0, kPolicyDevice);
          } else {
            uint64_t* d = reinterpret_cast<uint64_t*>(gout + dst[j]);
            __hip_atomic_store(d, (uint64_t)v[j][0] | ((uint64_t)v[j][1] << 32), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(d + 1, (uint64_t)v[j][2] | ((uint64_t)v[j][3] << 32), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    };
    using T1 = std::integral_constant<bool, true>;
    using F1 = std::integral_constant<bool, false>;
    if (one_shard && buf) copy(T1(), T1());
    else if (one_shard) copy(T1(), F1());
    else if (buf) copy(F1(), T1());
    else copy(F1(), F1());
  } else {  // 16-bit elements, any row length
    const int64_t n = rows * cols;
    for (int64_t i = threadIdx.x; i < n; i += kCopyThreads) {
      const int64_t R = row0 + i / cols, c = c0 + i % cols;
      const int64_t bb = R / a.block_rows, lr = R - bb * a.block_rows;
      __hip_atomic_store(gout + R * a.k + c, static_cast<const uint16_t*>(a.shards[bb])[lr * a.k + c],
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // Every thread waits for its own stores to complete -- they carry the
  // device-scope policy, so a completed store has been written through its
  // XCD's L2 and is visible device-wide -- then, after the barrier, one
  // thread raises the piece's flag (of the first raised_slabs slabs: a test
  // hook withholds the rest) with a relaxed system-scope store.  A release
  // fence or a release store would add an L2 write-back (buffer_wbl2) of
  // every dirty line of the XCD per workgroup: a 32 MB copy measured 36.6 us
  // with the fence against 15.2 us without (86.6 against 41.8 us after a
  // 512 MB write), and the release flag store alone still cost one
  // write-back per piece.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0 && sl < a.raised_slabs)
    __hip_atomic_store(a.flags + (int64_t)g * a.slabs + sl, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// One workgroup per piece.  (A fixed grid walking the pieces in order
// measured slower beside the GEMM: 142-155 us against 139 us.)
__global__ __launch_bounds__(kCopyThreads) void arrive_kernel(ArrivalArgs a) { copy_piece(a, (int)blockIdx.x); }

}  // namespace

hipError_t launch_arrival_copy(const ArrivalArgs& a, hipStream_t s) {
  const int64_t m = (int64_t)a.r * a.block_rows;
  if (a.r < 1 || a.r > kMaxRanks || a.block_rows < 1 || a.k < 1 || a.rows_chunk < 1 || a.slab_cols < 1 ||
      a.slabs < 1 || a.chunks < 1 || (int64_t)a.chunks * a.rows_chunk < m ||
      (int64_t)(a.chunks - 1) * a.rows_chunk >= m || (int64_t)a.slabs * a.slab_cols < a.k ||
      (int64_t)(a.slabs - 1) * a.slab_cols >= a.k || a.first_chunk < 0 || a.first_chunk >= a.chunks ||
      a.raised_slabs < 0 || a.raised_slabs > a.slabs)
    return hipErrorInvalidValue;
  arrive_kernel<<<(unsigned)((int64_t)a.chunks * a.slabs), kCopyThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mc2
