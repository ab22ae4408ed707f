// grad_bias of the tensor-parallel linear layer (hyper_parallel mc2.py,
// AllGatherMatmulFunction.backward and MatmulReduceScatterFunction.backward:
// grad_bias = grad_out.sum(dim=0)):
//
//   gb[j] = round16( sum over rows i of dy[i][j] )
//
// dy (m, n) 16-bit row-major.  A streaming column reduction bound by HBM
// (2 bytes read per element).  The sum runs in fp64: each 16-bit value has
// at most 11 significant bits, so a column's sum is exact as long as its
// values span fewer than about 53 - 11 - log2(m) binades (true for gradient
// data), and then does not depend on the order of the additions; it is
// rounded once (round to odd to fp32, then to nearest even to 16 bits,
// which equals one direct rounding).
//
// Vector path (n a multiple of 8): workgroup b owns one 16-byte column chunk
// (8 columns) over all rows, so no partial sums leave the workgroup.  Each
// of its 256 threads reads every 256th row, kBatch 16-byte loads in flight,
// and the threads' sums are combined through LDS in a fixed tree.  Workgroup
// b runs on XCD b % 8; the chunks are numbered so that each XCD owns a
// contiguous range of them, so the 8 chunks of a 128-byte line are mostly
// read by one XCD's L2.
#include "device.hpp"
#include "kernels.hpp"

namespace mc2 {
namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 8;

template <int DT>
__device__ __forceinline__ double dec16(uint32_t bits) {
  return DT == DT_BF16 ? (double)bf16_bits_to_f32(bits & 0xFFFFu) : (double)f16_bits_to_f32(bits & 0xFFFFu);
}
template <int DT>
__device__ __forceinline__ uint16_t round16(double v) {
  const float f = f64_to_f32_round_odd(v);
  return DT == DT_BF16 ? f32_to_bf16_bits(f) : f32_to_f16_bits(f);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void bias_grad_vec(const uint16_t* dy, int64_t m, int64_t n, uint16_t* gb) {
  __shared__ double red[kThreads][9];  // 9: odd pitch, no bank conflicts between threads
  const int64_t chunks = n / 8;
  int64_t c = blockIdx.x;
  if (chunks % 8 == 0) c = (blockIdx.x % 8) * (chunks / 8) + blockIdx.x / 8;
  const u32x4* src = reinterpret_cast<const u32x4*>(dy) + c;  // row i at src[i * chunks]
  double s[8];
#pragma unroll
  for (int e = 0; e < 8; e++) s[e] = 0.0;
  for (int64_t i0 = threadIdx.x; i0 < m; i0 += (int64_t)kBatch * kThreads) {
    u32x4 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; u++) {
      const int64_t i = i0 + (int64_t)u * kThreads;
      v[u] = i < m ? src[i * chunks] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kBatch; u++)
#pragma unroll
      for (int e = 0; e < 8; e++) s[e] += dec16<DT>(v[u][e / 2] >> (16 * (e & 1)));
  }
#pragma unroll
  for (int e = 0; e < 8; e++) red[threadIdx.x][e] = s[e];
  __syncthreads();
  for (int stride = kThreads / 2; stride > 0; stride /= 2) {
    if ((int)threadIdx.x < stride) {
#pragma unroll
      for (int e = 0; e < 8; e++) red[threadIdx.x][e] += red[threadIdx.x + stride][e];
    }
    __syncthreads();
  }
  if (threadIdx.x < 8) gb[c * 8 + threadIdx.x] = round16<DT>(red[0][threadIdx.x]);
}

// Any n: thread j of the grid sums column j over all rows (consecutive
// threads read consecutive columns of a row).
template <int DT>
__global__ __launch_bounds__(kThreads) void bias_grad_any(const uint16_t* dy, int64_t m, int64_t n, uint16_t* gb) {
  const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (j >= n) return;
  double s = 0.0;
  for (int64_t i = 0; i < m; i++) s += dec16<DT>(dy[i * n + j]);
  gb[j] = round16<DT>(s);
}

}  // namespace

hipError_t launch_bias_grad(const void* dy, int64_t m, int64_t n, int dtype, void* gb, hipStream_t s) {
  if (m < 1 || n < 1 || (dtype != DT_BF16 && dtype != DT_F16)) return hipErrorInvalidValue;
  const uint16_t* d = static_cast<const uint16_t*>(dy);
  uint16_t* o = static_cast<uint16_t*>(gb);
  if (n % 8 == 0) {
    const unsigned grid = (unsigned)(n / 8);
    if (dtype == DT_BF16) bias_grad_vec<DT_BF16><<<grid, kThreads, 0, s>>>(d, m, n, o);
    else bias_grad_vec<DT_F16><<<grid, kThreads, 0, s>>>(d, m, n, o);
  } else {
    const unsigned grid = (unsigned)((n + kThreads - 1) / kThreads);
    if (dtype == DT_BF16) bias_grad_any<DT_BF16><<<grid, kThreads, 0, s>>>(d, m, n, o);
    else bias_grad_any<DT_F16><<<grid, kThreads, 0, s>>>(d, m, n, o);
  }
  return hipGetLastError();
}

}  // namespace mc2
