// K1: 16-bit float GEMM on MFMA (v_mfma_f32_16x16x32_{bf16,f16}) with fp32
// accumulation and a single rounding of each output (the implementation the
// bf16 and fp16 translation units share), for
//   AllGatherMatmul  out = AllGather_m(shards) @ x2    (torch_npu
//                    npu_all_gather_base_mm page, "function" and "outputs")
//   dX_partial       = dY @ W                          (hyper_parallel mc2.py,
//   dW               = dY^T @ AllGather_m(X)            AllGatherMatmulFunction.backward)
//
// The tiling, LDS layout, transpose reads and XCD tile order are described
// in gemm_mfma.hpp.  Specific to this kernel:
//  - AllGather: A's row blocks are the rank shards, resolved per thread once
//    before the K loop, so the "communication" is the addressing of the
//    loads.  The gathered copy (gather_out) is written from the A tiles
//    already in LDS, each K step by one workgroup of the row of tiles (the
//    work spreads evenly): one write per element and no extra global read.
//  - Epilogue: fp32 -> bf16 / fp16 with round-to-nearest-even, staged through
//    LDS and stored as 16-byte row chunks.
//  - MatmulReduceScatter (hyper_parallel mc2.py, module docstring and
//    MatmulReduceScatterFunction.forward, Y = ReduceScatter_m(X @ W^T)): C is
//    this rank's partial.  The tiles of its own row block are handed out
//    last and store their rounded rows into the block output; the other rows
//    of C are the blocks it sends.  A streaming pass then sums the block
//    output with the blocks the other ranks sent, in rank order in fp32, and
//    rounds once.  Reducing inside the GEMM epilogue instead made every own
//    tile read seven scattered 256-byte row pieces per row at the same time,
//    well below streaming bandwidth; the separate pass reads whole rows.
#pragma once
#include <algorithm>

#include "gemm_mfma.hpp"

namespace mc2 {

// The 256 x 256 tile launches (gemm256.hip, its own translation unit: the
// 256 accumulator registers per lane of that tile need the AGPR form of the
// MFMAs, while the other tiles are built with their accumulators in VGPRs).
template <bool AK, bool BKM, int DT>
hipError_t launch_gemm16_256(const gemm::Problem& p, void* c, hipStream_t s);

namespace {

using namespace gemm;

template <int DT>
struct Ops16 {
  typedef f32x4 Acc;
  static __device__ __forceinline__ Acc mfma(u32x4 a, u32x4 b, Acc c) {
    if constexpr (DT == DT_BF16)
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint16_t cvt(float f) {
    return DT == DT_BF16 ? f32_to_bf16_bits(f) : f32_to_f16_bits(f);
  }
  static __device__ __forceinline__ float dec(uint32_t bits) {
    return DT == DT_BF16 ? bf16_bits_to_f32(bits & 0xFFFFu) : f16_bits_to_f32(bits & 0xFFFFu);
  }
};

// Reduce-scatter store of a staged tile (Problem::rs_out): the rows of the
// own block go to rs_out (row t of the block to rs_out row t), the others
// to C.  The rank-ordered sum with the received blocks follows in
// rs_reduce_kernel.
template <int BM, int BN, bool VEC>
__device__ __forceinline__ void store_rs_tile(const uint16_t* h0, const uint16_t* h1, uint16_t* C, const Problem& p,
                                              int64_t m0, int64_t n0) {
  constexpr int kRowChunks = BN / 8;
  const int64_t n = p.n;
  if constexpr (VEC && unrolled_store<BM, BN>()) {  // tile inside C: unrolled (as store_c16_tile)
    if (m0 + BM <= p.m && n0 + BN <= n) {
#pragma unroll 16
      for (int it = 0; it < BM * kRowChunks / kThreads; it++) {
        const int c = threadIdx.x + it * kThreads, row = c / kRowChunks, col = (c % kRowChunks) * 8;
        const int64_t grow = m0 + row, t = grow - p.rs_row0;
        const u32x4 v = *reinterpret_cast<const u32x4*>(staged_chunk<BM, BN>(h0, h1, row, col));
        if (t >= 0 && t < p.rs_rows) *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.rs_out) + t * n + n0 + col) = v;
        else store_out16(C + grow * n + n0 + col, v);
      }
      return;
    }
  }
  for (int c = threadIdx.x; c < BM * kRowChunks; c += kThreads) {
    const int row = c / kRowChunks, col = (c % kRowChunks) * 8;
    const int64_t grow = m0 + row, gcol = n0 + col;
    if (grow >= p.m) continue;
    const uint16_t* src = staged_chunk<BM, BN>(h0, h1, row, col);
    const int64_t t = grow - p.rs_row0;
    const bool own = t >= 0 && t < p.rs_rows;
    uint16_t* dst = own ? static_cast<uint16_t*>(p.rs_out) + t * n : C + grow * n;
    if (VEC && gcol + 8 <= n) {
      // rs_reduce_kernel reads the own block right after: plain stores keep it in the caches
      const u32x4 v = *reinterpret_cast<const u32x4*>(src);
      if (own) *reinterpret_cast<u32x4*>(dst + gcol) = v;
      else store_out16(dst + gcol, v);
    } else {
      for (int e = 0; e < 8; e++)
        if (gcol + e < n) dst[gcol + e] = src[e];
    }
  }
}

// The reduction of the own block, in place in rs_out: element e becomes
// round(B_0 + B_1 + ... + B_{ranks-1}) summed in fp32 in rank order, B_j =
// rs_recv[j][e] and B_rank = the rounded partial the GEMM left in rs_out.
// A streaming pass over whole rows (HBM-bound): 8 elements per thread and
// step, every block's load issued before the sum.
struct RsReduceArgs {
  uint16_t* out;
  const uint16_t* recv[kMaxRanks];  // own and unused slots: out
  const uint16_t* bias;             // (n) or NULL: added to the sum before the rounding
  int ranks;
  int64_t elems, n;
};

template <int DT, bool VEC>
__global__ __launch_bounds__(256) void rs_reduce_kernel(RsReduceArgs a) {
  using O = Ops16<DT>;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  if constexpr (VEC) {
    const int64_t chunks = a.elems / 8;
    for (int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; c < chunks; c += stride) {
      u32x4 v[kMaxRanks];
#pragma unroll
      for (int j = 0; j < kMaxRanks; j++) v[j] = reinterpret_cast<const u32x4*>(a.recv[j])[c];
      float sum[8];
#pragma unroll
      for (int j = 0; j < kMaxRanks; j++) {
        const bool used = j < a.ranks;
#pragma unroll
        for (int e = 0; e < 8; e++) {
          const float f = O::dec(v[j][e / 2] >> (16 * (e & 1)));
          sum[e] = j == 0 ? f : (used ? sum[e] + f : sum[e]);
        }
      }
      if (a.bias) {  // the chunk's 8 elements lie in one row (n % 8 == 0)
        const u32x4 b = *reinterpret_cast<const u32x4*>(a.bias + (c * 8) % a.n);
#pragma unroll
        for (int e = 0; e < 8; e++) sum[e] = sum[e] + O::dec(b[e / 2] >> (16 * (e & 1)));
      }
      u32x4 o;
#pragma unroll
      for (int w = 0; w < 4; w++) o[w] = (uint32_t)O::cvt(sum[2 * w]) | ((uint32_t)O::cvt(sum[2 * w + 1]) << 16);
      store_out16(reinterpret_cast<u32x4*>(a.out) + c, o);
    }
  } else {
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < a.elems; e += stride) {
      float sum = 0.0f;
      for (int j = 0; j < a.ranks; j++) sum = j == 0 ? O::dec(a.recv[j][e]) : sum + O::dec(a.recv[j][e]);
      if (a.bias) sum = sum + O::dec(a.bias[e % a.n]);
      a.out[e] = O::cvt(sum);
    }
  }
}

template <int DT>
hipError_t launch_rs_reduce(const GemmArgs& g, hipStream_t s) {
  RsReduceArgs a{};
  a.out = static_cast<uint16_t*>(g.rs_out);
  for (int j = 0; j < kMaxRanks; j++)
    a.recv[j] = (j < g.rs_ranks && j != g.rs_rank) ? static_cast<const uint16_t*>(g.rs_recv[j]) : a.out;
  a.bias = static_cast<const uint16_t*>(g.bias);
  a.ranks = g.rs_ranks;
  a.elems = g.rs_rows * g.n;
  a.n = g.n;
  // 16-byte chunks when every row of every block starts 16-byte aligned
  const bool vec = g.n % 8 == 0;
  const int64_t work = vec ? a.elems / 8 : a.elems;
  const int64_t blocks = std::min<int64_t>((work + 255) / 256, 256 * 16);
  if (vec) rs_reduce_kernel<DT, true><<<(unsigned)blocks, 256, 0, s>>>(a);
  else rs_reduce_kernel<DT, false><<<(unsigned)blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

// ARR: arrival emulation (A arrives in p.arrived piece by piece; gemm_mfma.hpp).
// GA: the call writes gather_out (the gather copy runs in the main loop).
template <int BM, int BN, bool AK, bool BKM, bool VEC, int DT, bool ARR, bool GA = false>
__global__ __launch_bounds__(kThreads, 1) void gemm16_kernel(Problem p, void* c) {
  constexpr int FM = BM / 32, FN = BN / 32;
  constexpr int NS = lds_stages<BM, BN>();
  __shared__ __attribute__((aligned(1024))) uint8_t s0[lds_stage_array_bytes<BM, BN>()];
  __shared__ __attribute__((aligned(1024))) uint8_t s1[lds_stage_array_bytes<BM, BN>()];
  __shared__ __attribute__((aligned(1024))) uint8_t s2[NS == 3 ? lds_stage_array_bytes<BM, BN>() : 16];
  int tm, tn;
  tile_of_block(p.m, p.n, BM, BN, p.tile_order_cols, p.tile_group, tm, tn, p.first_row_tile);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int tiles_n = (int)((p.n + BN - 1) / BN);

  typename Ops16<DT>::Acc acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the fused AllGatherMatmul loop with the gather copy walks K from a step
  // set by the tile (rot_start), as the gather-wavefront kernel does, so the
  // two give the same bits; arrival mode walks K in order, the order its
  // pieces arrive in, and so do the plain GEMMs (backward,
  // MatmulReduceScatter), which ran slower rotated
  run_mainloop<2, BM, BN, AK, BKM, VEC, ARR, NS, Ops16<DT>, GA ? 1 : 0, GA>(p, m0, n0, tn, tiles_n, s0, s1, s2, acc);

  uint16_t* h0 = reinterpret_cast<uint16_t*>(s0);
  uint16_t* h1 = reinterpret_cast<uint16_t*>(s1);
  // bias epilogue: three-stage tiles only (the 256 x 256 tile's registers are
  // all taken by its accumulators)
  if (lds_stages<BM, BN>() == 3 && p.bias) {
    // the lane's FN x 4 columns (accumulator layout: stage_c16), each bias
    // value loaded once
    constexpr int WN = BN / 2;
    const int lane = threadIdx.x % 64, wn = (threadIdx.x / 64) % 2;
    const uint16_t* bias = static_cast<const uint16_t*>(p.bias);
    float bv[FN][4];
#pragma unroll
    for (int j = 0; j < FN; j++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int64_t col = n0 + wn * WN + 16 * j + 4 * (lane / 16) + r;
        bv[j][r] = col < p.n ? Ops16<DT>::dec(bias[col]) : 0.0f;
      }
    stage_c16<BM, BN, DT>(h0, h1, [&](int i, int j, int r, int, int) { return acc[i][j][r] + bv[j][r]; });
  } else {
    stage_c16<BM, BN, DT>(h0, h1, [&](int i, int j, int r, int, int) { return acc[i][j][r]; });
  }
  if (p.rs_out) store_rs_tile<BM, BN, VEC>(h0, h1, static_cast<uint16_t*>(c), p, m0, n0);
  else store_c16_tile<BM, BN, VEC>(h0, h1, static_cast<uint16_t*>(c), p.m, p.n, m0, n0, !GA);
}

// AllGatherMatmul with gather_out on the fast path (A K-contiguous, three
// stages, no bias or arrival): 512 threads.  Wavefronts 0-3 run the GEMM's
// reads of the LDS stages and its MFMAs (mainloop_fast without loads);
// wavefronts 4-7 issue every load into the stages, wait for them before each
// barrier, and copy A tiles from the stages to gather_out (dma_waves_loop).
// The A tile of step kt sits in stage kt % 3 from the main loop's barrier kt
// (the prologue's counted as 0) until barrier kt + 1, after which the loads
// of step kt + 3 may overwrite it; the copy reads it in that window.  Both
// groups go through the same barriers (the loop's nk + 1, then the one that
// ends the staging of C).  The copy's stores count only in the loading
// wavefronts' vmcnt, and the GEMM wavefronts issue no global access in the
// loop at all (with the copy inside the GEMM's wavefronts every step that
// copies waited for its stores).  The workgroup of tile column tn copies the
// steps kt with kt % tiles_n == tn, so the tiles of a row share the copy of
// its A.  All 512 threads then store C.  AllGatherMatmul 8 x (512, 4096) @
// (4096, 1792), us: with its inputs in the caches 62.1 (copy in the GEMM's
// wavefronts) -> 55.0 (copy in wavefronts 4-7, loads in 0-3) -> 52.0 (loads
// also in 4-7; 51.9 without gather_out); after a 512 MB write 77.7 -> 77.1
// -> 77.8; in the benchmark step 72.4 -> 70.0 -> 70.0.  MC2_DMA_WAVES=0
// builds the variant with the loads in wavefronts 0-3.
#ifndef MC2_DMA_WAVES
#define MC2_DMA_WAVES 1
#endif

template <int BM, int BN, bool BKM, int DT>
__global__ __launch_bounds__(2 * kThreads, 1) void gemm16_gather_kernel(Problem p, void* c) {
  constexpr int FM = BM / 32, FN = BN / 32;
  constexpr int BK = kRowBytes / 2;
  static_assert(lds_stages<BM, BN>() == 3, "three stages");
  __shared__ __attribute__((aligned(1024))) uint8_t s0[lds_stage_array_bytes<BM, BN>()];
  __shared__ __attribute__((aligned(1024))) uint8_t s1[lds_stage_array_bytes<BM, BN>()];
  __shared__ __attribute__((aligned(1024))) uint8_t s2[lds_stage_array_bytes<BM, BN>()];
  int tm, tn;
  tile_of_block(p.m, p.n, BM, BN, p.tile_order_cols, p.tile_group, tm, tn, p.first_row_tile);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int tiles_n = (int)((p.n + BN - 1) / BN);
  uint16_t* h0 = reinterpret_cast<uint16_t*>(s0);
  uint16_t* h1 = reinterpret_cast<uint16_t*>(s1);
  if (threadIdx.x < kThreads) {
    typename Ops16<DT>::Acc acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
      for (int j = 0; j < FN; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the fast loop without the gather copy (the host launches this kernel
    // only where it applies)
#if MC2_DMA_WAVES
    run_loop_nodma<2, BM, BN, true, BKM, Ops16<DT>>(p, m0, n0, s0, s1, s2, acc);
#else
    run_fast_loop<2, BM, BN, true, BKM, Ops16<DT>>(p, m0, n0, s0, s1, s2, acc);
#endif
    stage_c16<BM, BN, DT>(h0, h1, [&](int i, int j, int r, int, int) { return acc[i][j][r]; });
  } else {
    const int tid = (int)threadIdx.x - kThreads;
#if MC2_DMA_WAVES
    dma_waves_loop<2, BM, BN, BKM>(p, m0, n0, tn, tiles_n, s0, s1, s2, tid);
#else
    const int nk = (int)(p.k / BK);
    int next = tn;
    for (int kt = 0; kt < nk; kt++) {
      lds_barrier();  // barrier kt: stage kt % 3 holds step kt
      if (kt == next) {
        const uint8_t* st = kt % 3 == 0 ? s0 : kt % 3 == 1 ? s1 : s2;
        copy_gather<2, BM>(st, p.gather_out, p.m, p.k, m0, (int64_t)kt * BK, tid);
        next += tiles_n;
      }
    }
    lds_barrier();   // barrier nk
#endif
    __syncthreads();  // the one that ends the staging of C
  }
  store_c16_tile<BM, BN, true, 2 * kThreads>(h0, h1, static_cast<uint16_t*>(c), p.m, p.n, m0, n0);
}

#ifndef MC2_GATHER_WAVES
#define MC2_GATHER_WAVES 1
#endif

template <int BM, int BN, bool AK, bool BKM, int DT>
hipError_t launch_cfg(Problem p, void* c, hipStream_t s) {
  const int64_t tiles = ((p.m + BM - 1) / BM) * ((p.n + BN - 1) / BN);
  // 16-byte vector access needs every row of every operand and of C to start
  // 16-byte aligned; the buffer-load staging needs operands below 2 GiB and
  // gathered row blocks of a multiple of 8 rows (otherwise: checked path)
  const int64_t a_bytes = AK ? (p.ready ? p.m : p.rows_per_part) * p.k * 2 : p.k * p.m * 2;
  const int parts = p.rows_per_part == p.m ? 1 : 2;
  const bool vec = (p.k % 8 == 0) && (AK || p.m % 8 == 0) && (p.n % 8 == 0) &&
                   dma_buffers_ok(a_bytes, p.k * p.n * 2, parts, p.rows_per_part) &&
                   dma_buffers_ok(p.rows_per_part * p.k * 2, 0, parts, p.rows_per_part);
  p.tile_order_cols = prefer_column_order(p.m, p.n, p.k, 2) ? 1 : 0;
  p.tile_group = choose_tile_group(p.m, p.n, BM, BN, p.tile_order_cols);
  if (p.rs_out) {  // own block last: start at the tile row after it
    const int64_t tiles_m = (p.m + BM - 1) / BM;
    p.first_row_tile = (int)(((p.rs_row0 + p.rs_rows) / BM) % tiles_m);
  }
  if constexpr (AK && lds_stages<BM, BN>() == 3) {
    if (p.ready) {
      if (vec) gemm16_kernel<BM, BN, AK, BKM, true, DT, true><<<(unsigned)tiles, kThreads, 0, s>>>(p, c);
      else gemm16_kernel<BM, BN, AK, BKM, false, DT, true><<<(unsigned)tiles, kThreads, 0, s>>>(p, c);
      return hipGetLastError();
    }
  }
  // the two-stage loop has neither the arrival wait nor the gather copy
  if (lds_stages<BM, BN>() == 2 && (p.ready || p.gather_out || p.bias)) return hipErrorInvalidValue;
  // (tiles of at most 128 x 224: the larger ones spill registers with 512 threads)
  if constexpr (MC2_GATHER_WAVES && AK && lds_stages<BM, BN>() == 3 && BM * BN <= 128 * 224) {
    // whole steps (the copy wavefronts count them as the fast loop does)
    if (p.gather_out && vec && !p.bias && !p.rs_out && p.k % 64 == 0 && p.kseg == p.k) {
      gemm16_gather_kernel<BM, BN, BKM, DT><<<(unsigned)tiles, 2 * kThreads, 0, s>>>(p, c);
      return hipGetLastError();
    }
  }
  if constexpr (AK && lds_stages<BM, BN>() == 3) {
    if (p.gather_out) {
      if (vec) gemm16_kernel<BM, BN, AK, BKM, true, DT, false, true><<<(unsigned)tiles, kThreads, 0, s>>>(p, c);
      else gemm16_kernel<BM, BN, AK, BKM, false, DT, false, true><<<(unsigned)tiles, kThreads, 0, s>>>(p, c);
      return hipGetLastError();
    }
  }
  if (vec) gemm16_kernel<BM, BN, AK, BKM, true, DT, false><<<(unsigned)tiles, kThreads, 0, s>>>(p, c);
  else gemm16_kernel<BM, BN, AK, BKM, false, DT, false><<<(unsigned)tiles, kThreads, 0, s>>>(p, c);
  return hipGetLastError();
}

// Tile shapes in order of preference among equal scores.  Of 256 x 128 and
// 128 x 256 (equal work per tile) the one with the narrower N-major operand
// comes first: that operand is read with transpose reads, which move fewer
// bytes per cycle than the K-major operand's 16-byte reads.  256 x 256 (two
// LDS stages) comes last and is used neither with the arrival wait nor with
// the gather copy: the first kNumTiles3 entries (three stages) serve those.
// It is left out with a K-contiguous A and an N-contiguous B: there the
// 256 x 128 tile measured faster (column-parallel dX: 129 against 137 us).
const TileChoice kTilesBN[] = {{128, 224}, {224, 128}, {256, 128}, {128, 256}, {128, 128}};  // A K-, B N-major
const TileChoice kTilesAM[] = {{128, 224}, {224, 128}, {128, 256}, {256, 128}, {128, 128}, {256, 256}};  // otherwise
constexpr int kNumTiles3 = 5;

template <bool AK, bool BKM>
constexpr const TileChoice* tiles16() { return (AK && !BKM) ? kTilesBN : kTilesAM; }
template <bool AK, bool BKM>
constexpr int num_tiles16() { return (AK && !BKM) ? 5 : 6; }

template <bool AK, bool BKM, int DT>
hipError_t launch_layout(const Problem& p, void* c, hipStream_t s) {
  // the arrival wait, the gather copy and the bias epilogue: three-stage tiles only
  const int count = (p.ready || p.gather_out || p.bias) ? kNumTiles3 : num_tiles16<AK, BKM>();
  const TileChoice t = tiles16<AK, BKM>()[pick_tile(p.m, p.n, tiles16<AK, BKM>(), count)];
  if (t.bm == 128 && t.bn == 224) return launch_cfg<128, 224, AK, BKM, DT>(p, c, s);
  if (t.bm == 224 && t.bn == 128) return launch_cfg<224, 128, AK, BKM, DT>(p, c, s);
  if (t.bm == 256 && t.bn == 128) return launch_cfg<256, 128, AK, BKM, DT>(p, c, s);
  if (t.bm == 128 && t.bn == 256) return launch_cfg<128, 256, AK, BKM, DT>(p, c, s);
  if constexpr (!(AK && !BKM))
    if (t.bm == 256 && t.bn == 256) return launch_gemm16_256<AK, BKM, DT>(p, c, s);
  return launch_cfg<128, 128, AK, BKM, DT>(p, c, s);
}

template <int DT>
hipError_t launch_dt(const GemmArgs& g, hipStream_t s) {
  Problem p{};
  for (int i = 0; i < kMaxRanks; i++) p.a_parts[i] = g.a_parts[i < g.num_parts ? i : 0];
  p.rows_per_part = g.rows_per_part;
  p.b = g.b;
  p.gather_out = g.gather_out;
  p.m = g.m;
  p.n = g.n;
  p.k = g.k;
  p.a_ld = g.k * 2;  // plain A: one K segment
  p.kseg = g.k;
  p.kseg_stride = 0;
  p.a_part_bytes = g.rows_per_part * g.k * 2;
  if (g.rs_out) {
    p.rs_out = g.rs_out;
    p.rs_row0 = g.rs_row0;
    p.rs_rows = g.rs_rows;
  } else {
    p.bias = g.bias;  // with rs_out the reduce-scatter pass adds it
  }
  if (g.ready_flags) {  // arrival emulation: A arrives in gather_out, which the kernel only reads
    p.ready = g.ready_flags;
    p.ready_value = g.ready_value;
    p.fallbacks = g.status_flag;
    p.wait_ticks = g.wait_ticks;
    p.arrived = g.gather_out;
    p.rows_chunk = g.rows_chunk;
    p.slab_cols = g.slab_cols;
    p.slabs = g.slabs;
    p.first_row_tile = g.first_row_tile;
    p.gather_out = nullptr;
  }
  if (g.a_kmajor && g.b_kmajor) return launch_layout<true, true, DT>(p, g.c, s);
  if (g.a_kmajor && !g.b_kmajor) return launch_layout<true, false, DT>(p, g.c, s);
  if (!g.a_kmajor && !g.b_kmajor) return launch_layout<false, false, DT>(p, g.c, s);
  return launch_layout<false, true, DT>(p, g.c, s);
}

}  // namespace

// One dtype's launches: the GEMM, then the reduce-scatter pass when asked for.
template <int DT>
hipError_t launch_gemm16_dt(const GemmArgs& g, hipStream_t s) {
  hipError_t e = launch_dt<DT>(g, s);
  if (e != hipSuccess || !g.rs_out) return e;
  return launch_rs_reduce<DT>(g, s);
}

}  // namespace mc2
