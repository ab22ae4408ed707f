// K1: 16-bit float GEMM on MFMA with fp32 accumulation, for
//   AllGatherMatmul  out = AllGather_m(shards) @ x2     (torch_npu
//                    npu_all_gather_base_mm page, "function"/"outputs")
//   dX_partial       = dY @ W                           (hyper_parallel mc2.py,
//   dW               = dY^T @ AllGather_m(X)             AllGatherMatmulFunction.backward)
//
// C (m, n) = A (m, k) @ B (k, n).  A is K-contiguous (row-major (m, k),
// possibly gathered from r row blocks that live in r separate buffers) or
// M-contiguous (stored (k, m)); B is K-contiguous (stored (n, k)) or
// N-contiguous (row-major (k, n)).
//
// Workgroup: 256 threads = 4 wavefronts in a 2 x 2 grid; each wavefront owns
// a (BM/2) x (BN/2) block of C as 16 x 16 MFMA tiles
// (v_mfma_f32_16x16x32_{bf16,f16}).  Operand tiles go global -> registers ->
// LDS, double buffered, so the loads of step k+1 are in flight while the
// MFMAs of step k run.  In LDS a K-contiguous operand is stored [mn][k]
// and its MFMA fragments are read with 16-byte ds_read_b128; an
// MN-contiguous operand is stored [k][mn] as loaded and its fragments come
// from ds_read_b64_tr_b16, the gfx950 LDS transpose read: in each 16-lane
// group lane t reads 4 elements of row k0 + t/4 at column n0 + 4 (t % 4), and
// receives column n0 + t of rows k0 .. k0+3.
//
// Gather: the row block of gathered row r is r / rows_per_part, so A is read
// straight from the shard buffers.  The workgroups of column tile 0 also
// store the A chunks they load into gather_out, which therefore costs no
// extra reads.
#include "device.hpp"
#include "kernels.hpp"

namespace mc2 {
namespace {

constexpr int kThreads = 256;
constexpr int kPad = 8;  // elements of padding per LDS row (16 bytes)

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <int DT>
struct Frag;
template <>
struct Frag<DT_BF16> {
  typedef bf16x8 type;
  static __device__ __forceinline__ f32x4 mfma(type a, type b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint16_t cvt(float f) { return f32_to_bf16_bits(f); }
};
template <>
struct Frag<DT_F16> {
  typedef f16x8 type;
  static __device__ __forceinline__ f32x4 mfma(type a, type b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint16_t cvt(float f) { return f32_to_f16_bits(f); }
};

// A tile of R (mn) x BK (k) elements of one operand.
//   KMAJ: global element (mn, k) at base[mn * ld + k], LDS [R][BK + kPad]
//  !KMAJ: global element (mn, k) at base[k * ld + mn], LDS [BK][R + kPad]
// Loads are 8-element (16-byte) chunks; each thread owns CH chunks.
template <int R, int BK, bool KMAJ>
struct TileShape {
  static constexpr int kChunks = R * BK / 8;
  static constexpr int kPerThread = kChunks / kThreads;
  static constexpr int kLdsElems = KMAJ ? R * (BK + kPad) : BK * (R + kPad);
  static_assert(kChunks % kThreads == 0, "tile must split evenly into 16-byte chunks");
};

struct OperandSrc {
  const uint16_t* parts[kMaxRanks];
  int64_t rows_per_part;  // gathered operand: row block size (== mn extent if one part)
  int64_t ld;             // leading dimension in elements
  int64_t mn_extent, k_extent;
};

// Chunk c of a tile -> (mn, k) offsets inside the tile.
template <int R, int BK, bool KMAJ>
__device__ __forceinline__ void chunk_coords(int c, int& mn, int& k) {
  if constexpr (KMAJ) {
    mn = c / (BK / 8);
    k = (c % (BK / 8)) * 8;
  } else {
    k = c / (R / 8);
    mn = (c % (R / 8)) * 8;
  }
}

template <int R, int BK, bool KMAJ, bool VEC>
__device__ __forceinline__ void load_tile(const OperandSrc& src, int64_t mn0, int64_t k0,
                                          u32x4 (&regs)[TileShape<R, BK, KMAJ>::kPerThread],
                                          uint16_t* gather_out) {
  using TS = TileShape<R, BK, KMAJ>;
#pragma unroll
  for (int i = 0; i < TS::kPerThread; i++) {
    const int c = threadIdx.x + i * kThreads;
    int mn, k;
    chunk_coords<R, BK, KMAJ>(c, mn, k);
    const int64_t gmn = mn0 + mn, gk = k0 + k;
    u32x4 v = {0u, 0u, 0u, 0u};
    if constexpr (KMAJ) {
      if (gmn < src.mn_extent) {
        const int64_t part = gmn / src.rows_per_part;
        const uint16_t* row = src.parts[part] + (gmn - part * src.rows_per_part) * src.ld;
        if (VEC && gk + 8 <= src.k_extent) {
          v = *reinterpret_cast<const u32x4*>(row + gk);
          if (gather_out) *reinterpret_cast<u32x4*>(gather_out + gmn * src.k_extent + gk) = v;
        } else {
          uint16_t e[8];
#pragma unroll
          for (int j = 0; j < 8; j++) e[j] = (gk + j < src.k_extent) ? row[gk + j] : (uint16_t)0;
#pragma unroll
          for (int j = 0; j < 4; j++) v[j] = (uint32_t)e[2 * j] | ((uint32_t)e[2 * j + 1] << 16);
          if (gather_out) {
#pragma unroll
            for (int j = 0; j < 8; j++)
              if (gk + j < src.k_extent) gather_out[gmn * src.k_extent + gk + j] = e[j];
          }
        }
      }
    } else {
      if (gk < src.k_extent) {
        const uint16_t* row = src.parts[0] + gk * src.ld;
        if (VEC && gmn + 8 <= src.mn_extent) {
          v = *reinterpret_cast<const u32x4*>(row + gmn);
        } else {
          uint16_t e[8];
#pragma unroll
          for (int j = 0; j < 8; j++) e[j] = (gmn + j < src.mn_extent) ? row[gmn + j] : (uint16_t)0;
#pragma unroll
          for (int j = 0; j < 4; j++) v[j] = (uint32_t)e[2 * j] | ((uint32_t)e[2 * j + 1] << 16);
        }
      }
    }
    regs[i] = v;
  }
}

template <int R, int BK, bool KMAJ>
__device__ __forceinline__ void store_tile(uint16_t* lds, const u32x4 (&regs)[TileShape<R, BK, KMAJ>::kPerThread]) {
  using TS = TileShape<R, BK, KMAJ>;
#pragma unroll
  for (int i = 0; i < TS::kPerThread; i++) {
    const int c = threadIdx.x + i * kThreads;
    int mn, k;
    chunk_coords<R, BK, KMAJ>(c, mn, k);
    const int off = KMAJ ? mn * (BK + kPad) + k : k * (R + kPad) + mn;
    *reinterpret_cast<u32x4*>(lds + off) = regs[i];
  }
}

// MFMA fragment of 16 (mn) x 32 (k) at tile offsets (mn0, k0): lane l gets
// the 8 k values 8 (l / 16) .. +7 of row mn0 + l % 16.
template <int R, int BK, bool KMAJ, int DT>
__device__ __forceinline__ typename Frag<DT>::type read_frag(const uint16_t* lds, int mn0, int k0) {
  const int l = threadIdx.x % 64;
  if constexpr (KMAJ) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(lds + (mn0 + l % 16) * (BK + kPad) + k0 + 8 * (l / 16));
    return __builtin_bit_cast(typename Frag<DT>::type, v);
  } else {
    const int t = l % 16, g = l / 16;
    const uint16_t* p0 = lds + (k0 + 8 * g + t / 4) * (R + kPad) + mn0 + 4 * (t % 4);
    const uint16_t* p1 = p0 + 4 * (R + kPad);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p1);
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(typename Frag<DT>::type, v);
  }
}

template <int BM, int BN, int BK, bool AK, bool BKM, bool VEC, int DT>
__global__ __launch_bounds__(kThreads) void gemm16_kernel(GemmArgs g) {
  using TA = TileShape<BM, BK, AK>;
  using TB = TileShape<BN, BK, BKM>;
  constexpr int WM = BM / 2, WN = BN / 2;   // wavefront block
  constexpr int FM = WM / 16, FN = WN / 16; // MFMA tiles per wavefront
  constexpr int kStage = TA::kLdsElems + TB::kLdsElems;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kStage];

  const int tiles_n = (int)((g.n + BN - 1) / BN);
  const int tile_m = blockIdx.x / tiles_n, tile_n = blockIdx.x % tiles_n;
  const int64_t m0 = (int64_t)tile_m * BM, n0 = (int64_t)tile_n * BN;

  OperandSrc sa, sb;
  for (int i = 0; i < kMaxRanks; i++) sa.parts[i] = static_cast<const uint16_t*>(i < g.num_parts ? g.a_parts[i] : g.a_parts[0]);
  sa.rows_per_part = g.rows_per_part;
  sa.ld = AK ? g.k : g.m;
  sa.mn_extent = g.m;
  sa.k_extent = g.k;
  sb.parts[0] = static_cast<const uint16_t*>(g.b);
  for (int i = 1; i < kMaxRanks; i++) sb.parts[i] = sb.parts[0];
  sb.rows_per_part = g.n;
  sb.ld = BKM ? g.k : g.n;
  sb.mn_extent = g.n;
  sb.k_extent = g.k;
  uint16_t* gout = (AK && tile_n == 0) ? static_cast<uint16_t*>(g.gather_out) : nullptr;

  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int wm = wave / 2, wn = wave % 2;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[TA::kPerThread], rb[TB::kPerThread];
  const int nk = (int)((g.k + BK - 1) / BK);
  load_tile<BM, BK, AK, VEC>(sa, m0, 0, ra, gout);
  load_tile<BN, BK, BKM, VEC>(sb, n0, 0, rb, nullptr);
  store_tile<BM, BK, AK>(lds, ra);
  store_tile<BN, BK, BKM>(lds + TA::kLdsElems, rb);
  __syncthreads();

  for (int kt = 0; kt < nk; kt++) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      load_tile<BM, BK, AK, VEC>(sa, m0, (int64_t)(kt + 1) * BK, ra, gout);
      load_tile<BN, BK, BKM, VEC>(sb, n0, (int64_t)(kt + 1) * BK, rb, nullptr);
    }
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      typename Frag<DT>::type fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; i++) fa[i] = read_frag<BM, BK, AK, DT>(lds + cur * kStage, wm * WM + 16 * i, kk);
#pragma unroll
      for (int j = 0; j < FN; j++) fb[j] = read_frag<BN, BK, BKM, DT>(lds + cur * kStage + TA::kLdsElems, wn * WN + 16 * j, kk);
#pragma unroll
      for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++) acc[i][j] = Frag<DT>::mfma(fa[i], fb[j], acc[i][j]);
    }
    if (kt + 1 < nk) {
      store_tile<BM, BK, AK>(lds + (cur ^ 1) * kStage, ra);
      store_tile<BN, BK, BKM>(lds + (cur ^ 1) * kStage + TA::kLdsElems, rb);
    }
    __syncthreads();
  }

  uint16_t* C = static_cast<uint16_t*>(g.c);
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++) {
      const int64_t col = n0 + wn * WN + 16 * j + lane % 16;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int64_t row = m0 + wm * WM + 16 * i + 4 * (lane / 16) + r;
        if (row < g.m && col < g.n) C[row * g.n + col] = Frag<DT>::cvt(acc[i][j][r]);
      }
    }
}

template <int BM, int BN, int BK, bool AK, bool BKM, int DT>
hipError_t launch_cfg(const GemmArgs& g, hipStream_t s) {
  const int64_t tiles = ((g.m + BM - 1) / BM) * ((g.n + BN - 1) / BN);
  // 16-byte vector loads need every row of every operand to start 16-byte aligned
  const bool vec = (g.k % 8 == 0) && (AK || g.m % 8 == 0) && (BKM || g.n % 8 == 0);
  if (vec) gemm16_kernel<BM, BN, BK, AK, BKM, true, DT><<<(unsigned)tiles, kThreads, 0, s>>>(g);
  else gemm16_kernel<BM, BN, BK, AK, BKM, false, DT><<<(unsigned)tiles, kThreads, 0, s>>>(g);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const GemmArgs& g, hipStream_t s) {
  if (g.a_kmajor && g.b_kmajor) return launch_cfg<128, 128, 64, true, true, DT>(g, s);
  if (g.a_kmajor && !g.b_kmajor) return launch_cfg<128, 128, 64, true, false, DT>(g, s);
  if (!g.a_kmajor && !g.b_kmajor) return launch_cfg<128, 128, 64, false, false, DT>(g, s);
  return launch_cfg<128, 128, 64, false, true, DT>(g, s);
}

}  // namespace

hipError_t launch_gemm16(const GemmArgs& g, hipStream_t s) {
  if (g.m < 1 || g.n < 1 || g.k < 1 || g.num_parts < 1 || g.num_parts > kMaxRanks) return hipErrorInvalidValue;
  if (g.num_parts * g.rows_per_part != g.m) return hipErrorInvalidValue;
  if (g.gather_out && !g.a_kmajor) return hipErrorInvalidValue;
  if (g.dtype == DT_BF16) return launch_dt<DT_BF16>(g, s);
  if (g.dtype == DT_F16) return launch_dt<DT_F16>(g, s);
  return hipErrorInvalidValue;
}

}  // namespace mc2
