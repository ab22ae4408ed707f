// K3: int8 GEMM with exact int32 accumulation and the fused dequant epilogue
// of AlltoAllQuantMatmul (aclnnAlltoAllQuantMatmul page, "function"
// formulas: output_quant = permutedOut_quant @ x2; output = output_quant *
// x1_scale * x2_scale; output = output + bias).
//
//   out[i][j] = round16( (float(acc[i][j]) * s1[i]) * s2[j] + bias[j] )
//
// A = q (m, k) int8 row-major (K-contiguous), B = x2 (k, n) int8 row-major
// (N-contiguous).  Workgroup: 256 threads = 4 wavefronts in a 2 x 2 grid,
// each owning a (BM/2) x (BN/2) block of C as 16 x 16 tiles of
// v_mfma_i32_16x16x64_i8.  Operand tiles go global -> registers -> LDS,
// double buffered.  A's fragments are read with ds_read_b128 from a [m][k]
// LDS tile; B stays [k][n] in LDS and its fragments come from the gfx950
// transpose read ds_read_b64_tr_b8 (in each 16-lane group lane t reads 8
// bytes of row k0 + t/2 at column n0 + 8 (t % 2) and receives column n0 + t
// of rows k0 .. k0+7).  Integer accumulation is exact, so the result does not
// depend on the order of the K loop.
#include "device.hpp"
#include "kernels.hpp"

namespace mc2 {
namespace {

constexpr int kThreads = 256;
constexpr int kPadB = 16;  // bytes of padding per LDS row

typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2;

template <int R, int BK, bool KMAJ>
struct TileShapeI8 {
  static constexpr int kChunks = R * BK / 16;
  static constexpr int kPerThread = kChunks / kThreads;
  static constexpr int kLdsBytes = KMAJ ? R * (BK + kPadB) : BK * (R + kPadB);
  static_assert(kChunks % kThreads == 0, "tile must split evenly into 16-byte chunks");
};

template <int R, int BK, bool KMAJ>
__device__ __forceinline__ void chunk_coords8(int c, int& mn, int& k) {
  if constexpr (KMAJ) {
    mn = c / (BK / 16);
    k = (c % (BK / 16)) * 16;
  } else {
    k = c / (R / 16);
    mn = (c % (R / 16)) * 16;
  }
}

// KMAJ: element (mn, k) at base[mn * ld + k]; else at base[k * ld + mn].
template <int R, int BK, bool KMAJ, bool VEC>
__device__ __forceinline__ void load_tile8(const int8_t* base, int64_t ld, int64_t mn_ext, int64_t k_ext,
                                           int64_t mn0, int64_t k0,
                                           u32x4 (&regs)[TileShapeI8<R, BK, KMAJ>::kPerThread]) {
  using TS = TileShapeI8<R, BK, KMAJ>;
#pragma unroll
  for (int i = 0; i < TS::kPerThread; i++) {
    const int c = threadIdx.x + i * kThreads;
    int mn, k;
    chunk_coords8<R, BK, KMAJ>(c, mn, k);
    const int64_t gmn = mn0 + mn, gk = k0 + k;
    u32x4 v = {0u, 0u, 0u, 0u};
    if constexpr (KMAJ) {
      if (gmn < mn_ext) {
        const int8_t* row = base + gmn * ld;
        if (VEC && gk + 16 <= k_ext) {
          v = *reinterpret_cast<const u32x4*>(row + gk);
        } else {
#pragma unroll
          for (int j = 0; j < 16; j++)
            if (gk + j < k_ext) v[j / 4] |= ((uint32_t)(uint8_t)row[gk + j]) << (8 * (j % 4));
        }
      }
    } else {
      if (gk < k_ext) {
        const int8_t* row = base + gk * ld;
        if (VEC && gmn + 16 <= mn_ext) {
          v = *reinterpret_cast<const u32x4*>(row + gmn);
        } else {
#pragma unroll
          for (int j = 0; j < 16; j++)
            if (gmn + j < mn_ext) v[j / 4] |= ((uint32_t)(uint8_t)row[gmn + j]) << (8 * (j % 4));
        }
      }
    }
    regs[i] = v;
  }
}

template <int R, int BK, bool KMAJ>
__device__ __forceinline__ void store_tile8(uint8_t* lds, const u32x4 (&regs)[TileShapeI8<R, BK, KMAJ>::kPerThread]) {
  using TS = TileShapeI8<R, BK, KMAJ>;
#pragma unroll
  for (int i = 0; i < TS::kPerThread; i++) {
    const int c = threadIdx.x + i * kThreads;
    int mn, k;
    chunk_coords8<R, BK, KMAJ>(c, mn, k);
    const int off = KMAJ ? mn * (BK + kPadB) + k : k * (R + kPadB) + mn;
    *reinterpret_cast<u32x4*>(lds + off) = regs[i];
  }
}

// 16 (mn) x 64 (k) fragment: lane l gets k = 16 (l / 16) .. +15 of row mn0 + l % 16.
template <int R, int BK, bool KMAJ>
__device__ __forceinline__ i32x4 read_frag8(const uint8_t* lds, int mn0, int k0) {
  const int l = threadIdx.x % 64;
  if constexpr (KMAJ) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(lds + (mn0 + l % 16) * (BK + kPadB) + k0 + 16 * (l / 16));
    return __builtin_bit_cast(i32x4, v);
  } else {
    const int t = l % 16, g = l / 16;
    const uint8_t* p0 = lds + (k0 + 16 * g + t / 2) * (R + kPadB) + mn0 + 8 * (t % 2);
    const uint8_t* p1 = p0 + 8 * (R + kPadB);
    const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)p0));
    const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)p1));
    const i32x4 v = {(int)lo[0], (int)lo[1], (int)hi[0], (int)hi[1]};
    return v;
  }
}

template <int BM, int BN, int BK, bool VEC, int DT>
__global__ __launch_bounds__(kThreads) void gemm_i8_kernel(GemmI8Args g) {
  using TA = TileShapeI8<BM, BK, true>;
  using TB = TileShapeI8<BN, BK, false>;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int kStage = TA::kLdsBytes + TB::kLdsBytes;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStage];

  const int tiles_n = (int)((g.n + BN - 1) / BN);
  const int tile_m = blockIdx.x / tiles_n, tile_n = blockIdx.x % tiles_n;
  const int64_t m0 = (int64_t)tile_m * BM, n0 = (int64_t)tile_n * BN;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int wm = wave / 2, wn = wave % 2;

  i32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++) acc[i][j] = i32x4{0, 0, 0, 0};

  u32x4 ra[TA::kPerThread], rb[TB::kPerThread];
  const int nk = (int)((g.k + BK - 1) / BK);
  load_tile8<BM, BK, true, VEC>(g.a, g.k, g.m, g.k, m0, 0, ra);
  load_tile8<BN, BK, false, VEC>(g.b, g.n, g.n, g.k, n0, 0, rb);
  store_tile8<BM, BK, true>(lds, ra);
  store_tile8<BN, BK, false>(lds + TA::kLdsBytes, rb);
  __syncthreads();

  for (int kt = 0; kt < nk; kt++) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      load_tile8<BM, BK, true, VEC>(g.a, g.k, g.m, g.k, m0, (int64_t)(kt + 1) * BK, ra);
      load_tile8<BN, BK, false, VEC>(g.b, g.n, g.n, g.k, n0, (int64_t)(kt + 1) * BK, rb);
    }
#pragma unroll
    for (int kk = 0; kk < BK; kk += 64) {
      i32x4 fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; i++) fa[i] = read_frag8<BM, BK, true>(lds + cur * kStage, wm * WM + 16 * i, kk);
#pragma unroll
      for (int j = 0; j < FN; j++) fb[j] = read_frag8<BN, BK, false>(lds + cur * kStage + TA::kLdsBytes, wn * WN + 16 * j, kk);
#pragma unroll
      for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++) acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      store_tile8<BM, BK, true>(lds + (cur ^ 1) * kStage, ra);
      store_tile8<BN, BK, false>(lds + (cur ^ 1) * kStage + TA::kLdsBytes, rb);
    }
    __syncthreads();
  }

  const uint16_t* bias = static_cast<const uint16_t*>(g.bias);
  uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++) {
      const int64_t col = n0 + wn * WN + 16 * j + lane % 16;
      if (col >= g.n) continue;
      const float s2 = g.s2[col];
      float b = 0.0f;
      if (bias) b = DT == DT_BF16 ? bf16_bits_to_f32(bias[col]) : f16_bits_to_f32(bias[col]);
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int64_t row = m0 + wm * WM + 16 * i + 4 * (lane / 16) + r;
        if (row >= g.m) continue;
        const int32_t a = acc[i][j][r];
        float v = (float)a * g.s1[row];
        v = v * s2;
        v = v + b;
        out[row * g.n + col] = DT == DT_BF16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v);
        if (g.acc_out) g.acc_out[row * g.n + col] = a;
      }
    }
}

template <int DT>
hipError_t launch_dt(const GemmI8Args& g, hipStream_t s) {
  constexpr int BM = 128, BN = 128, BK = 128;
  const int64_t tiles = ((g.m + BM - 1) / BM) * ((g.n + BN - 1) / BN);
  const bool vec = (g.k % 16 == 0) && (g.n % 16 == 0);
  if (vec) gemm_i8_kernel<BM, BN, BK, true, DT><<<(unsigned)tiles, kThreads, 0, s>>>(g);
  else gemm_i8_kernel<BM, BN, BK, false, DT><<<(unsigned)tiles, kThreads, 0, s>>>(g);
  return hipGetLastError();
}

}  // namespace

size_t gemm_i8_workspace_bytes(int64_t, int64_t, int64_t) { return 256; }

hipError_t launch_gemm_i8(const GemmI8Args& g, hipStream_t s) {
  if (g.m < 1 || g.n < 1 || g.k < 1) return hipErrorInvalidValue;
  if (g.dtype == DT_BF16) return launch_dt<DT_BF16>(g, s);
  if (g.dtype == DT_F16) return launch_dt<DT_F16>(g, s);
  return hipErrorInvalidValue;
}

}  // namespace mc2
