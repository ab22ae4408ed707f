// libmc2 C ABI: host-side validation, device checks and kernel dispatch.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>
#include <string>

#include "api_internal.hpp"
#include "kernels.hpp"
#include "mc2.h"
#include "testing.h"
#include "validate.hpp"

namespace mc2 {
namespace {

constexpr int kMaxDevices = 64;

struct DeviceState {
  bool checked = false;
  bool ok = false;
  // arrival emulation: copy stream, fork / join events, ready flags (one per
  // rank block, then the fallback counter) and a call counter that makes
  // every call's flag value new
  bool arrival_ready = false;
  hipStream_t copy_stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  unsigned* flags = nullptr;
  unsigned epoch = 0;
  // held from recording `fork` on a caller's stream to waiting on `join`, so
  // calls from several host threads do not re-record the shared events in
  // between
  std::mutex fork_mutex;
};
DeviceState g_dev[kMaxDevices];
std::mutex g_dev_mutex;

// Arrival test hook (testing.h): the GEMM's wait limit and how many leading
// slabs of K the copy raises flags for (negative: all).
std::atomic<uint64_t> g_arrival_wait_ticks{kArrivalWaitTicks};
std::atomic<int> g_arrival_raised_slabs{-1};

mc2_status hip_fail(hipError_t e, const char* where) {
  return fail(MC2_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

int dt(mc2_dtype d) { return static_cast<int>(d); }

// Arrival flags: up to kArrivalFlags (row chunk, slab) pieces, then the
// count of timed-out waits.
constexpr int64_t kArrivalSlabs = 16;
constexpr int64_t kArrivalFlags = 65535;
constexpr int kFallbackSlot = (int)kArrivalFlags;
constexpr size_t kFlagBytes = (kArrivalFlags + 1) * sizeof(unsigned);

// Creates the arrival-emulation resources of device `dev` once.  The flags
// sit in uncached device memory so that the GEMM's polls read memory, not a
// stale cache line; that memory is kept until the process ends.
// *epoch receives this call's flag value (never 0, the flags' initial value),
// taken under the lock so concurrent callers get distinct values.
mc2_status arrival_setup(int dev, DeviceState** out, unsigned* epoch = nullptr) {
  std::lock_guard<std::mutex> lock(g_dev_mutex);
  DeviceState& st = g_dev[dev];
  if (!st.arrival_ready) {
    hipError_t e = hipStreamCreateWithFlags(&st.copy_stream, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&st.fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&st.join, hipEventDisableTiming);
    if (e == hipSuccess)
      e = hipExtMallocWithFlags(reinterpret_cast<void**>(&st.flags), kFlagBytes, hipDeviceMallocUncached);
    if (e == hipSuccess) e = hipMemset(st.flags, 0, kFlagBytes);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "arrival emulation set-up");
    st.arrival_ready = true;
  }
  if (epoch) {
    if (++st.epoch == 0) ++st.epoch;
    *epoch = st.epoch;
  }
  *out = &st;
  return MC2_OK;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

#ifndef MC2_PREFETCH_SIDE
#define MC2_PREFETCH_SIDE 1
#endif

// The int8 GEMM (K3) with its weight's pass through the last-level cache
// (K9, prefetch.hip).  With the device's side stream (side != NULL), K9 runs
// beside K3 instead of before it: it streams the weight ahead of the GEMM's
// K loop from the CU slots K3 leaves free, and `st` waits for it only after
// K3, so it is off the critical path.  Without (the no-allocation entry
// point, which creates no stream), K9 runs first on `st`.
mc2_status gemm_i8_prefetched(const GemmI8Args& ga, int64_t w_bytes, DeviceState* side, hipStream_t st,
                              const char* where) {
  hipError_t e;
  if (side) {
    std::lock_guard<std::mutex> fork_lock(side->fork_mutex);
    e = hipEventRecord(side->fork, st);
    if (e == hipSuccess) e = launch_gemm_i8(ga, st);
    if (e == hipSuccess) e = hipStreamWaitEvent(side->copy_stream, side->fork, 0);
    if (e == hipSuccess) e = launch_prefetch(ga.b, w_bytes, side->copy_stream);
    if (e == hipSuccess) e = hipEventRecord(side->join, side->copy_stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(st, side->join, 0);
  } else {
    e = launch_prefetch(ga.b, w_bytes, st);
    if (e == hipSuccess) e = launch_gemm_i8(ga, st);
  }
  if (e != hipSuccess) return hip_fail(e, where);
  return MC2_OK;
}

}  // namespace

// The current device must be a gfx950 (MI355X class) GPU.
mc2_status current_device(int* dev_out) {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count < 1) {
    (void)hipGetLastError();
    return fail(MC2_ERR_NO_DEVICE, "no HIP device");
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MC2_ERR_NO_DEVICE, "device index out of range");
  std::lock_guard<std::mutex> lock(g_dev_mutex);
  DeviceState& st = g_dev[dev];
  if (!st.checked) {
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    st.ok = std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
    st.checked = true;
  }
  if (!st.ok) return fail(MC2_ERR_NO_DEVICE, "the current device is not gfx950");
  *dev_out = dev;
  return MC2_OK;
}

// The A16W8 chain with a caller-provided workspace (the two public entry
// points differ only in where the workspace comes from).
mc2_status alltoall_quant_matmul_run(const void* x1, int rank_size, int64_t bs, int64_t h, mc2_dtype x1_dtype,
                                     const int8_t* x2, int64_t n, const float* x2_scale, const void* x1_smooth,
                                     const void* bias, void* out, void* permuted_out, int8_t* q_out,
                                     float* x1_scale_out, int32_t* acc_out, void* workspace,
                                     size_t workspace_bytes, void* stream, bool device_checked, bool w4) {
  size_t need = 0;
  mc2_status s = mc2_alltoall_quant_matmul_workspace_size(rank_size, bs, h, n, &need);
  if (s != MC2_OK) {
    if (s == MC2_ERR_SHAPE && (!x1 || !x2 || !x2_scale || !out))
      return fail(MC2_ERR_NULL, "alltoall_quant_matmul: x1, x2, x2_scale and out are required");
    return s;
  }
  // A16W4: N even (two int4 codes per byte along N)
  if (w4 && n % 2 != 0) return fail(MC2_ERR_SHAPE, "alltoall_quant_matmul_a16w4: n must be even");
  const int64_t rows = bs / rank_size, cols = (int64_t)rank_size * h;
  s = check_alltoall_quant_matmul(x1, rank_size, bs, h, x1_dtype, x2, n, x2_scale, x1_smooth, bias, out,
                                  permuted_out, q_out, x1_scale_out, acc_out, workspace, workspace_bytes,
                                  w4 ? need + (size_t)(cols * n) : need);
  if (s != MC2_OK) return s;
  int dev;
  if (!device_checked && (s = current_device(&dev)) != MC2_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int8_t* x2w = reinterpret_cast<int8_t*>(ws + need);  // A16W4: the widened weight, past the A16W8 part
  int8_t* q = q_out ? q_out : reinterpret_cast<int8_t*>(ws);
  ws += align_up((size_t)(rows * cols), 256);
  float* s1 = x1_scale_out ? x1_scale_out : reinterpret_cast<float*>(ws);
  ws += align_up((size_t)rows * 4, 256);

  QuantArgs qa{};
  qa.x1 = x1;
  qa.smooth = x1_smooth;
  qa.q = q;
  qa.s1 = s1;
  qa.permuted = permuted_out;
  qa.bs = bs;
  qa.h = h;
  qa.r = rank_size;
  qa.dtype = dt(x1_dtype);
  hipError_t e = launch_permute_quant(qa, st);
  if (e != hipSuccess) return hip_fail(e, "alltoall_quant_matmul quant launch");
  // The weight passes through the caches just before or while the GEMM reads
  // it: A16W4 widens it (int4 -> int8) after the quantisation, A16W8 streams it
  // once (K9) beside the GEMM (gemm_i8_prefetched).  (K9 on the side stream
  // beside K2, with the GEMM waiting for both, measured slower: both kernels
  // slowed down and the join before the GEMM cost about 11 us.)
  if (w4) {
    WidenArgs wa{};
    wa.src[0] = reinterpret_cast<const uint8_t*>(x2);
    wa.dst[0] = x2w;
    wa.bytes[0] = cols * n / 2;
    e = launch_widen_int4(wa, st);
    if (e != hipSuccess) return hip_fail(e, "alltoall_quant_matmul_a16w4 widening launch");
    x2 = x2w;
  }

  GemmI8Args ga{};
  ga.a = q;
  ga.b = x2;
  ga.s1 = s1;
  ga.s2 = x2_scale;
  ga.bias = bias;
  ga.out = out;
  ga.acc_out = acc_out;
  ga.m = rows;
  ga.n = n;
  ga.k = cols;
  ga.dtype = dt(x1_dtype);
  ga.partials = reinterpret_cast<int32_t*>(ws);
  if (w4) {
    e = launch_gemm_i8(ga, st);
    if (e != hipSuccess) return hip_fail(e, "alltoall_quant_matmul gemm launch");
    return MC2_OK;
  }
  // the side stream is set up once per device; the no-allocation entry point
  // (device_checked) creates none and runs K9 first
  DeviceState* side = nullptr;
  if (MC2_PREFETCH_SIDE && !device_checked && (s = arrival_setup(dev, &side)) != MC2_OK) return s;
  return gemm_i8_prefetched(ga, cols * n, side, st, "alltoall_quant_matmul gemm launch");
}

}  // namespace mc2

using namespace mc2;

extern "C" {

const char* mc2_status_string(mc2_status s) {
  switch (s) {
    case MC2_OK: return "MC2_OK";
    case MC2_ERR_NULL: return "MC2_ERR_NULL: a required pointer is NULL";
    case MC2_ERR_SHAPE: return "MC2_ERR_SHAPE: a size breaks the operator's constraints";
    case MC2_ERR_DTYPE: return "MC2_ERR_DTYPE: dtype not supported";
    case MC2_ERR_UNSUPPORTED: return "MC2_ERR_UNSUPPORTED: not provided by this library";
    case MC2_ERR_WORKSPACE: return "MC2_ERR_WORKSPACE: workspace missing or too small";
    case MC2_ERR_NO_DEVICE: return "MC2_ERR_NO_DEVICE: no gfx950 device";
    case MC2_ERR_HIP: return "MC2_ERR_HIP: HIP runtime error";
    case MC2_ERR_ALIGN: return "MC2_ERR_ALIGN: tensor pointer not 16-byte aligned";
  }
  return "unknown mc2_status";
}

const char* mc2_last_error(void) { return last_error_text(); }

mc2_status mc2_quant_all_reduce(const void* const* x, const void* const* scales, int world_size,
                                int64_t rows, int64_t h, mc2_dtype x_dtype,
                                mc2_dtype scale_dtype, void* out, mc2_dtype out_dtype,
                                void* stream) {
  clear_error();
  mc2_status s = check_quant_all_reduce(x, scales, world_size, rows, h, x_dtype, scale_dtype, out, out_dtype);
  if (s != MC2_OK) return s;
  int dev;
  if ((s = current_device(&dev)) != MC2_OK) return s;
  QarArgs a{};
  for (int i = 0; i < world_size; i++) {
    a.x[i] = x[i];
    a.scales[i] = scales[i];
  }
  a.out = out;
  a.total = rows * h;
  a.h = h;
  a.r = world_size;
  a.x_dtype = dt(x_dtype);
  a.scale_dtype = dt(scale_dtype);
  a.out_dtype = dt(out_dtype);
  hipError_t e = launch_dequant_sum(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "quant_all_reduce launch");
  return MC2_OK;
}

mc2_status mc2_quant_reduce_scatter(const void* const* x, const void* const* scales, int world_size, int rank_id,
                                    int64_t rows, int64_t h, mc2_dtype x_dtype, mc2_dtype scale_dtype, void* out,
                                    mc2_dtype out_dtype, void* stream) {
  clear_error();
  mc2_status s = check_quant_reduce_scatter(x, scales, world_size, rank_id, rows, h, x_dtype, scale_dtype, out,
                                            out_dtype);
  if (s != MC2_OK) return s;
  int dev;
  if ((s = current_device(&dev)) != MC2_OK) return s;
  // this rank's rows of the sum: the same pass over its row block of every input
  const int64_t block = rows / world_size, row0 = (int64_t)rank_id * block;
  const int64_t scale_row_bytes = scale_dtype == MC2_F32 ? (h / 128) * 4 : h / 32;
  QarArgs a{};
  for (int i = 0; i < world_size; i++) {
    a.x[i] = static_cast<const uint8_t*>(x[i]) + row0 * h;
    a.scales[i] = static_cast<const uint8_t*>(scales[i]) + row0 * scale_row_bytes;
  }
  a.out = out;
  a.total = block * h;
  a.h = h;
  a.r = world_size;
  a.x_dtype = dt(x_dtype);
  a.scale_dtype = dt(scale_dtype);
  a.out_dtype = dt(out_dtype);
  hipError_t e = launch_dequant_sum(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "quant_reduce_scatter launch");
  return MC2_OK;
}

mc2_status mc2_matmul_grad_input(const void* dy, const void* w, int64_t m, int64_t n_local,
                                 int64_t k, mc2_dtype dtype, void* dx_partial, void* stream) {
  clear_error();
  mc2_status s = check_grad_input(dy, w, m, n_local, k, dtype, dx_partial);
  if (s != MC2_OK) return s;
  int dev;
  if ((s = current_device(&dev)) != MC2_OK) return s;
  GemmArgs a{};
  a.a_parts[0] = dy;  // A = dY (m, n_local), K-contiguous
  a.num_parts = 1;
  a.rows_per_part = m;
  a.a_kmajor = 1;
  a.b = w;            // B = W (n_local, k): (k_contract, n) row-major
  a.b_kmajor = 0;
  a.c = dx_partial;
  a.m = m;
  a.n = k;
  a.k = n_local;
  a.dtype = dt(dtype);
  hipError_t e = launch_gemm16(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "matmul_grad_input launch");
  return MC2_OK;
}

}  // extern "C"

namespace mc2 {
namespace {

// MatmulReduceScatter share with an optional bias added to the reduced block.
mc2_status matmul_reduce_scatter_impl(const void* x, const void* x2, int world_size, int rank_id, int64_t m,
                                      int64_t k, int64_t n, int x2_trans, mc2_dtype dtype, const void* const* recv,
                                      const void* bias, void* out, void* partial_out, void* stream) {
  mc2_status s = check_matmul_reduce_scatter(x, x2, world_size, rank_id, m, k, n, dtype, recv, out, partial_out);
  if (s != MC2_OK) return s;
  int dev;
  if ((s = current_device(&dev)) != MC2_OK) return s;
  GemmArgs a{};
  a.a_parts[0] = x;  // A = x (m, k), K-contiguous
  a.num_parts = 1;
  a.rows_per_part = m;
  a.a_kmajor = 1;
  a.b = x2;          // (k, n) row-major, or (n, k) row-major with x2_trans
  a.b_kmajor = x2_trans ? 1 : 0;
  a.c = partial_out;
  a.m = m;
  a.n = n;
  a.k = k;
  a.dtype = dt(dtype);
  a.rs_out = out;
  for (int j = 0; j < world_size; j++) a.rs_recv[j] = j == rank_id ? nullptr : recv[j];
  a.rs_ranks = world_size;
  a.rs_rank = rank_id;
  a.rs_rows = m / world_size;
  a.rs_row0 = (int64_t)rank_id * a.rs_rows;
  a.bias = bias;
  hipError_t e = launch_gemm16(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "matmul_reduce_scatter launch");
  return MC2_OK;
}

}  // namespace
}  // namespace mc2

extern "C" {

mc2_status mc2_matmul_reduce_scatter(const void* x, const void* x2, int world_size, int rank_id, int64_t m,
                                     int64_t k, int64_t n, int x2_trans, mc2_dtype dtype, const void* const* recv,
                                     void* out, void* partial_out, void* stream) {
  clear_error();
  return matmul_reduce_scatter_impl(x, x2, world_size, rank_id, m, k, n, x2_trans, dtype, recv, nullptr, out,
                                    partial_out, stream);
}

mc2_status mc2_matmul_reduce_scatter_bias(const void* x, const void* x2, int world_size, int rank_id, int64_t m,
                                          int64_t k, int64_t n, int x2_trans, mc2_dtype dtype,
                                          const void* const* recv, const void* bias, void* out, void* partial_out,
                                          void* stream) {
  clear_error();
  mc2_status s = check_bias("matmul_reduce_scatter_bias", bias);
  if (s != MC2_OK) return s;
  return matmul_reduce_scatter_impl(x, x2, world_size, rank_id, m, k, n, x2_trans, dtype, recv, bias, out,
                                    partial_out, stream);
}

mc2_status mc2_matmul_grad_weight(const void* dy, const void* ag_x, int64_t m, int64_t n_local,
                                  int64_t k, mc2_dtype dtype, void* dw, void* stream) {
  clear_error();
  mc2_status s = check_grad_weight(dy, ag_x, m, n_local, k, dtype, dw);
  if (s != MC2_OK) return s;
  int dev;
  if ((s = current_device(&dev)) != MC2_OK) return s;
  GemmArgs a{};
  a.a_parts[0] = dy;  // A = dY^T: dy (m, n_local) is A stored transposed
  a.num_parts = 1;
  a.rows_per_part = n_local;
  a.a_kmajor = 0;
  a.b = ag_x;         // B = AG(X) (m, k): (k_contract, n) row-major
  a.b_kmajor = 0;
  a.c = dw;
  a.m = n_local;
  a.n = k;
  a.k = m;
  a.dtype = dt(dtype);
  hipError_t e = launch_gemm16(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "matmul_grad_weight launch");
  return MC2_OK;
}

}  // extern "C"

namespace mc2 {
namespace {

// AllGatherMatmul with an optional bias added before the output's rounding.
mc2_status allgather_matmul_impl(const void* const* shards, int world_size, int64_t m_local, int64_t k,
                                 const void* x2, int64_t n, int x2_trans, mc2_dtype dtype, const void* bias,
                                 void* out, void* gather_out, mc2_ag_mode mode, int rank_id, void* stream) {
  mc2_status s = check_allgather_matmul(shards, world_size, m_local, k, x2, n, dtype, out, gather_out,
                                        static_cast<int>(mode), rank_id);
  if (s != MC2_OK) return s;
  int dev;
  if ((s = current_device(&dev)) != MC2_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  GemmArgs a{};
  a.rows_per_part = m_local;
  a.a_kmajor = 1;
  a.b = x2;
  a.b_kmajor = x2_trans ? 1 : 0;
  a.c = out;
  a.m = (int64_t)world_size * m_local;
  a.n = n;
  a.k = k;
  a.dtype = dt(dtype);
  a.bias = bias;
  if (mode == MC2_AG_FUSED_WRITE) {
    for (int i = 0; i < world_size; i++) a.a_parts[i] = shards[i];
    a.num_parts = world_size;
    a.gather_out = gather_out;
    hipError_t e = launch_gemm16(a, st);
    if (e != hipSuccess) return hip_fail(e, "allgather_matmul launch");
    return MC2_OK;
  }
  // Arrival emulation.  Fork a copy stream off `stream`; on it a copy kernel
  // fills gather_out piece by piece (row chunks of the GEMM's tile height or
  // a multiple of it, times up to 16 slabs of K), local rank's rows first,
  // each piece followed by its ready flag (= this call's epoch).  The GEMM on
  // `stream` reads A from gather_out and issues the loads of each slab of K
  // once its piece has arrived.  `stream` then joins the copy stream, so work
  // enqueued after this call sees the whole gather_out.
  DeviceState* ds = nullptr;
  unsigned epoch = 0;
  if ((s = arrival_setup(dev, &ds, &epoch)) != MC2_OK) return s;
  const int64_t m = a.m;
  int64_t slabs = (k + 63) / 64 < kArrivalSlabs ? (k + 63) / 64 : kArrivalSlabs;
  const int64_t slab_cols = ((k + slabs - 1) / slabs + 63) / 64 * 64;
  slabs = (k + slab_cols - 1) / slab_cols;
  int64_t rows_chunk = gemm16_tile_rows(m, n, a.b_kmajor);
  while (((m + rows_chunk - 1) / rows_chunk) * slabs > kArrivalFlags) rows_chunk *= 2;
  const int64_t chunks = (m + rows_chunk - 1) / rows_chunk;
  const int64_t first_chunk = (int64_t)rank_id * m_local / rows_chunk;
  ArrivalArgs c{};
  for (int i = 0; i < world_size; i++) c.shards[i] = shards[i];
  c.gather_out = gather_out;
  c.flags = ds->flags;
  c.block_rows = m_local;
  c.k = k;
  c.rows_chunk = rows_chunk;
  c.slab_cols = slab_cols;
  c.slabs = (int)slabs;
  const int raised = g_arrival_raised_slabs.load();
  c.raised_slabs = raised < 0 || raised > slabs ? (int)slabs : raised;
  c.chunks = (int)chunks;
  c.r = world_size;
  c.first_chunk = (int)first_chunk;
  c.epoch = epoch;
  std::lock_guard<std::mutex> fork_lock(ds->fork_mutex);
  hipError_t e = hipEventRecord(ds->fork, st);
  if (e == hipSuccess) e = hipStreamWaitEvent(ds->copy_stream, ds->fork, 0);
  if (e == hipSuccess) e = launch_arrival_copy(c, ds->copy_stream);
  if (e != hipSuccess) return hip_fail(e, "allgather_matmul arrival copy");
  for (int i = 0; i < world_size; i++) a.a_parts[i] = shards[i];
  a.num_parts = world_size;
  a.gather_out = gather_out;
  a.ready_flags = ds->flags;
  a.ready_value = epoch;
  a.rows_chunk = rows_chunk;
  a.slab_cols = slab_cols;
  a.slabs = (int)slabs;
  a.first_row_tile = (int)(first_chunk * rows_chunk / gemm16_tile_rows(m, n, a.b_kmajor));
  a.status_flag = ds->flags + kFallbackSlot;
  a.wait_ticks = g_arrival_wait_ticks.load();
  e = launch_gemm16(a, st);
  if (e == hipSuccess) e = hipEventRecord(ds->join, ds->copy_stream);
  if (e == hipSuccess) e = hipStreamWaitEvent(st, ds->join, 0);
  if (e != hipSuccess) return hip_fail(e, "allgather_matmul arrival launch");
  return MC2_OK;
}

}  // namespace
}  // namespace mc2

extern "C" {

mc2_status mc2_allgather_matmul(const void* const* shards, int world_size, int64_t m_local,
                                int64_t k, const void* x2, int64_t n, int x2_trans,
                                mc2_dtype dtype, void* out, void* gather_out, mc2_ag_mode mode,
                                int rank_id, void* stream) {
  clear_error();
  return allgather_matmul_impl(shards, world_size, m_local, k, x2, n, x2_trans, dtype, nullptr, out, gather_out,
                               mode, rank_id, stream);
}

mc2_status mc2_allgather_matmul_bias(const void* const* shards, int world_size, int64_t m_local, int64_t k,
                                     const void* x2, int64_t n, int x2_trans, mc2_dtype dtype, const void* bias,
                                     void* out, void* gather_out, mc2_ag_mode mode, int rank_id, void* stream) {
  clear_error();
  mc2_status s = check_bias("allgather_matmul_bias", bias);
  if (s != MC2_OK) return s;
  return allgather_matmul_impl(shards, world_size, m_local, k, x2, n, x2_trans, dtype, bias, out, gather_out,
                               mode, rank_id, stream);
}

mc2_status mc2_bias_grad(const void* dy, int64_t m, int64_t n, mc2_dtype dtype, void* grad_bias, void* stream) {
  clear_error();
  mc2_status s = check_bias_grad(dy, m, n, dtype, grad_bias);
  if (s != MC2_OK) return s;
  int dev;
  if ((s = current_device(&dev)) != MC2_OK) return s;
  hipError_t e = launch_bias_grad(dy, m, n, dt(dtype), grad_bias, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "bias_grad launch");
  return MC2_OK;
}

mc2_status mc2_allgather_arrival_fallbacks(int reset, unsigned* count) {
  clear_error();
  if (!count) return fail(MC2_ERR_NULL, "allgather_arrival_fallbacks: count is NULL");
  int dev;
  mc2_status s = current_device(&dev);
  if (s != MC2_OK) return s;
  DeviceState* ds = nullptr;
  if ((s = arrival_setup(dev, &ds)) != MC2_OK) return s;
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(count, ds->flags + kFallbackSlot, sizeof(unsigned), hipMemcpyDeviceToHost);
  if (e == hipSuccess && reset) e = hipMemset(ds->flags + kFallbackSlot, 0, sizeof(unsigned));
  if (e == hipSuccess && reset) e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "allgather_arrival_fallbacks");
  return MC2_OK;
}

mc2_status mc2_testing_arrival(uint64_t wait_ticks, int raised_slabs) {
  clear_error();
  g_arrival_wait_ticks.store(wait_ticks ? wait_ticks : kArrivalWaitTicks);
  g_arrival_raised_slabs.store(raised_slabs);
  return MC2_OK;
}

mc2_status mc2_alltoall_quant_matmul_workspace_size(int rank_size, int64_t bs, int64_t h,
                                                    int64_t n, size_t* bytes) {
  clear_error();
  if (!bytes) return fail(MC2_ERR_NULL, "workspace_size: bytes is NULL");
  mc2_status s = check_alltoall_sizes(rank_size, bs, h, n);
  if (s != MC2_OK) return s;
  const int64_t rows = bs / rank_size, cols = (int64_t)rank_size * h;
  *bytes = align_up((size_t)(rows * cols), 256) + align_up((size_t)rows * 4, 256) +
           gemm_i8_workspace_bytes(rows, n, cols);
  return MC2_OK;
}

mc2_status mc2_alltoall_quant_matmul(const void* x1, int rank_size, int64_t bs, int64_t h,
                                     mc2_dtype x1_dtype, const int8_t* x2, int64_t n,
                                     const float* x2_scale, const void* x1_smooth,
                                     const void* bias, void* out, void* permuted_out,
                                     int8_t* q_out, float* x1_scale_out, int32_t* acc_out,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  return alltoall_quant_matmul_run(x1, rank_size, bs, h, x1_dtype, x2, n, x2_scale, x1_smooth, bias, out,
                                   permuted_out, q_out, x1_scale_out, acc_out, workspace, workspace_bytes, stream,
                                   false);
}

mc2_status mc2_alltoall_quant_matmul_a16w4(const void* x1, int rank_size, int64_t bs, int64_t h,
                                           mc2_dtype x1_dtype, const uint8_t* x2, int64_t n, const float* x2_scale,
                                           const void* x1_smooth, const void* bias, void* out, void* permuted_out,
                                           int8_t* q_out, float* x1_scale_out, int32_t* acc_out, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  clear_error();
  return alltoall_quant_matmul_run(x1, rank_size, bs, h, x1_dtype, reinterpret_cast<const int8_t*>(x2), n, x2_scale,
                                   x1_smooth, bias, out, permuted_out, q_out, x1_scale_out, acc_out, workspace,
                                   workspace_bytes, stream, false, true);
}

mc2_status mc2_alltoall_quant_matmul_a16w4_workspace_size(int rank_size, int64_t bs, int64_t h, int64_t n,
                                                          size_t* bytes) {
  clear_error();
  if (!bytes) return fail(MC2_ERR_NULL, "a16w4_workspace_size: bytes is NULL");
  size_t need = 0;
  mc2_status s = mc2_alltoall_quant_matmul_workspace_size(rank_size, bs, h, n, &need);
  if (s != MC2_OK) return s;
  if (n % 2 != 0) return fail(MC2_ERR_SHAPE, "a16w4_workspace_size: n must be even");
  *bytes = need + (size_t)rank_size * (size_t)h * (size_t)n;
  return MC2_OK;
}

mc2_status mc2_alltoall_quant_matmul_a4w4_workspace_size(int rank_size, int64_t bs, int64_t h, int64_t n,
                                                         size_t* bytes) {
  clear_error();
  if (!bytes) return fail(MC2_ERR_NULL, "a4w4_workspace_size: bytes is NULL");
  mc2_status s = check_alltoall_a4w4_sizes(rank_size, bs, h, n);
  if (s != MC2_OK) return s;
  *bytes = align_up((size_t)(bs * h), 256) + (size_t)rank_size * (size_t)h * (size_t)n;
  return MC2_OK;
}

mc2_status mc2_alltoall_quant_matmul_a4w4(const uint8_t* x1, int rank_size, int64_t bs, int64_t h,
                                          const float* x1_scale, const uint8_t* x2, int64_t n,
                                          const float* x2_scale, const void* bias, void* out, mc2_dtype out_dtype,
                                          int32_t* acc_out, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  mc2_status s = check_alltoall_a4w4(x1, rank_size, bs, h, x1_scale, x2, n, x2_scale, bias, out, out_dtype, acc_out);
  if (s != MC2_OK) return s;
  const size_t x1w_bytes = align_up((size_t)(bs * h), 256);
  const size_t need = x1w_bytes + (size_t)rank_size * (size_t)h * (size_t)n;
  if (!workspace || workspace_bytes < need)
    return fail(MC2_ERR_WORKSPACE, "alltoall_quant_matmul_a4w4: workspace needs " + std::to_string(need) + " bytes");
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return fail(MC2_ERR_ALIGN, "alltoall_quant_matmul_a4w4: workspace not 16-byte aligned");
  int dev;
  if ((s = current_device(&dev)) != MC2_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // both operands widened to int8 (x1 first, then x2, in the workspace),
  // then the int8 chain of the static entry point
  int8_t* x1w = static_cast<int8_t*>(workspace);
  int8_t* x2w = x1w + x1w_bytes;
  WidenArgs wa{};
  wa.src[0] = x1;
  wa.dst[0] = x1w;
  wa.bytes[0] = bs * h / 2;
  wa.src[1] = x2;
  wa.dst[1] = x2w;
  wa.bytes[1] = (int64_t)rank_size * h * n / 2;
  hipError_t e = launch_widen_int4(wa, st);
  if (e != hipSuccess) return hip_fail(e, "alltoall_quant_matmul_a4w4 widening launch");
  // The AlltoAll permute is the GEMM's addressing of A (as in the static
  // entry point): K split into rank_size segments of h codes, (bs / rank_size) h apart.
  const int64_t rows = bs / rank_size, cols = (int64_t)rank_size * h;
  GemmI8Args ga{};
  ga.a = x1w;
  ga.a_ld = h;
  ga.kseg = h;
  ga.kseg_stride = rows * h;
  ga.a_bytes = bs * h;
  ga.b = x2w;
  ga.s1 = x1_scale;
  ga.s2 = x2_scale;
  ga.bias = bias;
  ga.out = out;
  ga.acc_out = acc_out;
  ga.m = rows;
  ga.n = n;
  ga.k = cols;
  ga.dtype = dt(out_dtype);
  e = launch_gemm_i8(ga, st);
  if (e != hipSuccess) return hip_fail(e, "alltoall_quant_matmul_a4w4 launch");
  return MC2_OK;
}

mc2_status mc2_alltoall_quant_matmul_static(const int8_t* x1, int rank_size, int64_t bs, int64_t h,
                                            const float* x1_scale, const int8_t* x2, int64_t n,
                                            const float* x2_scale, const void* bias, void* out,
                                            mc2_dtype out_dtype, int8_t* permuted_out, int32_t* acc_out,
                                            void* stream) {
  clear_error();
  mc2_status s = check_alltoall_quant_matmul_static(x1, rank_size, bs, h, x1_scale, x2, n, x2_scale, bias, out,
                                                    out_dtype, permuted_out, acc_out);
  if (s != MC2_OK) return s;
  int dev;
  if ((s = current_device(&dev)) != MC2_OK) return s;
  // The AlltoAll permute is the GEMM's addressing of A: row t of P is the r
  // segments x1[(j T + t) h : + h], j = 0..r-1, so A = x1 with K split into
  // r segments of h elements, T h bytes apart.
  const int64_t rows = bs / rank_size, cols = (int64_t)rank_size * h;
  GemmI8Args ga{};
  ga.a = x1;
  ga.a_ld = h;
  ga.kseg = h;
  ga.kseg_stride = rows * h;
  ga.a_bytes = bs * h;
  ga.permuted_out = permuted_out;
  ga.b = x2;
  ga.s1 = x1_scale;
  ga.s2 = x2_scale;
  ga.bias = bias;
  ga.out = out;
  ga.acc_out = acc_out;
  ga.m = rows;
  ga.n = n;
  ga.k = cols;
  ga.dtype = dt(out_dtype);
  DeviceState* side = nullptr;
  if (MC2_PREFETCH_SIDE && (s = arrival_setup(dev, &side)) != MC2_OK) return s;
  return gemm_i8_prefetched(ga, cols * n, side, static_cast<hipStream_t>(stream), "alltoall_quant_matmul_static launch");
}

}  // extern "C"
