// Tiled MFMA GEMM shared by K1 (16-bit float) and K3 (int8) on gfx950.
//
// C (m, n) = A (m, k) @ B (k, n) with 1- or 2-byte elements.  A is either
// K-contiguous ((m, k) row-major, possibly gathered from up to 8 row blocks
// held in separate buffers) or M-contiguous (stored (k, m)); B is either
// K-contiguous (stored (n, k)) or N-contiguous ((k, n) row-major).
//
// Geometry is the same for both element sizes when counted in bytes: a
// K step of the main loop covers 128 bytes of K, an MFMA consumes 64 bytes of
// K per lane group (v_mfma_f32_16x16x32_{bf16,f16}: 32 elements;
// v_mfma_i32_16x16x64_i8: 64 elements), every global load and LDS write is a
// 16-byte chunk, and every MFMA operand fragment is 16 bytes per lane.
//
// Workgroup: 256 threads = 4 wavefronts in a 2 x 2 grid; each wavefront owns a
// (BM/2) x (BN/2) block of C as 16 x 16 MFMA tiles.  Operand tiles go global ->
// registers -> LDS, double buffered: the global loads of step k+1 are issued
// before the MFMAs of step k and written to the other LDS buffer after them,
// with one barrier per step.  In LDS a K-contiguous operand is stored [mn][k]
// and its fragments are read with ds_read_b128; an MN-contiguous operand is
// stored [k][mn] exactly as loaded and its fragments come from the gfx950
// transpose reads (within each 16-lane group):
//   ds_read_b64_tr_b16: lane t reads 4 elements of row k0 + t/4 at column
//                       n0 + 4 (t % 4) and receives column n0 + t of rows k0..k0+3
//   ds_read_b64_tr_b8:  lane t reads 8 bytes of row k0 + t/2 at column
//                       n0 + 8 (t % 2) and receives column n0 + t of rows k0..k0+7
// LDS rows are padded (see kPadBytesK / kPadBytesMN) against bank conflicts.
//
// Tile order: workgroup b is dispatched to XCD b % 8.  Tiles are renumbered so
// each XCD owns a contiguous 1/8 of them, walking along rows of tiles (the
// XCD's L2 shares A and streams B) or along columns (shares B), whichever
// makes the L2s fetch fewer bytes in total.
#pragma once
#include <type_traits>

#include "device.hpp"
#include "kernels.hpp"

namespace mc2 {
namespace gemm {

constexpr int kThreads = 256;
constexpr int kBKBytes = 128;   // K bytes per main-loop step
// LDS row padding: 32 bytes for [mn][k] tiles (a 160-byte pitch makes the
// 16-lane ds_read_b128 fragment reads conflict-free; 144 does not), 16 bytes
// for [k][mn] tiles (any pitch that is not a multiple of 256 bytes serves the
// transpose reads equally).
constexpr int kPadBytesK = 32;
constexpr int kPadBytesMN = 16;

typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// One operand tile: R (mn) x BK (k) elements of E bytes, in 16-byte chunks.
template <int E, int R, bool KMAJ>
struct Tile {
  static constexpr int kCh = 16 / E;                 // elements per chunk
  static constexpr int kBK = kBKBytes / E;           // K elements per step
  static constexpr int kPad = (KMAJ ? kPadBytesK : kPadBytesMN) / E;  // padding in elements
  static constexpr int kPitch = KMAJ ? kBK + kPad : R + kPad;
  static constexpr int kLds = KMAJ ? R * kPitch : kBK * kPitch;  // elements
  static constexpr int kChunks = R * kBK / kCh;
  static constexpr int kPer = kChunks / kThreads;
  static_assert(kChunks % kThreads == 0, "tile must split evenly into 16-byte chunks");
  static __device__ __forceinline__ void coords(int c, int& mn, int& k) {
    if constexpr (KMAJ) {
      mn = c / (kBK / kCh);
      k = (c % (kBK / kCh)) * kCh;
    } else {
      k = c / (R / kCh);
      mn = (c % (R / kCh)) * kCh;
    }
  }
  static __device__ __forceinline__ int lds_off(int mn, int k) { return KMAJ ? mn * kPitch + k : k * kPitch + mn; }
};

template <int E>
struct Elem;
template <>
struct Elem<2> { typedef uint16_t T; };
template <>
struct Elem<1> { typedef uint8_t T; };

template <typename T, int N>
struct VecOf {
  typedef T type __attribute__((ext_vector_type(N)));
};

// Per-thread view of one operand: the source of each of its chunks.
template <int E, int R, bool KMAJ>
struct Loader {
  using TS = Tile<E, R, KMAJ>;
  using T = typename Elem<E>::T;
  const T* ptr[TS::kPer];  // chunk source at k = 0
  int64_t ld, k_ext, mn_ext, mn0;
  T* gout;  // copy of what is loaded (gather_out), K-contiguous A only

  // tile coordinates of chunk i of this thread (recomputed, not stored, to save registers)
  static __device__ __forceinline__ int kofs(int i) {
    int mn, k;
    TS::coords(threadIdx.x + i * kThreads, mn, k);
    return k;
  }
  static __device__ __forceinline__ int mnofs(int i) {
    int mn, k;
    TS::coords(threadIdx.x + i * kThreads, mn, k);
    return mn;
  }
  __device__ __forceinline__ bool mn_ok(int i) const { return mn0 + mnofs(i) < mn_ext; }

  __device__ __forceinline__ void init(const void* const* parts, int64_t rows_per_part, int64_t ld_,
                                       int64_t mn_ext_, int64_t k_ext_, int64_t mn0_, void* gather_out) {
    ld = ld_;
    k_ext = k_ext_;
    mn_ext = mn_ext_;
    mn0 = mn0_;
    gout = static_cast<T*>(gather_out);
#pragma unroll
    for (int i = 0; i < TS::kPer; i++) {
      int mn, k;
      TS::coords(threadIdx.x + i * kThreads, mn, k);
      const int64_t gmn = mn0 + mn;
      if constexpr (KMAJ) {
        // row blocks of rows_per_part rows live in separate buffers
        int part = 0;
        int64_t local = gmn < mn_ext ? gmn : 0;
        while (local >= rows_per_part) {
          local -= rows_per_part;
          part++;
        }
        ptr[i] = static_cast<const T*>(parts[part]) + local * ld + k;
      } else {
        ptr[i] = static_cast<const T*>(parts[0]) + (int64_t)k * ld + gmn;
      }
    }
  }

  // Loads the chunks of the K step starting at k0.  When the whole tile lies
  // inside the matrix (the common case, decided uniformly per workgroup) the
  // loads carry no bounds checks, so they issue back to back.
  template <bool VEC>
  __device__ __forceinline__ void load(int64_t k0, u32x4 (&regs)[TS::kPer]) const {
    constexpr int CH = TS::kCh;
    const bool full = VEC && (mn0 + R <= mn_ext) && (k0 + TS::kBK <= k_ext);
    if (full) {
#pragma unroll
      for (int i = 0; i < TS::kPer; i++)
        regs[i] = *reinterpret_cast<const u32x4*>(KMAJ ? ptr[i] + k0 : ptr[i] + k0 * ld);
      return;
    }
#pragma unroll
    for (int i = 0; i < TS::kPer; i++) {
      const int64_t gk = k0 + kofs(i);
      u32x4 v = {0u, 0u, 0u, 0u};
      if constexpr (KMAJ) {
        const T* p = ptr[i] + k0;
        if (VEC) {
          if (mn_ok(i) && gk + CH <= k_ext) v = *reinterpret_cast<const u32x4*>(p);
        } else if (mn_ok(i)) {
          T e[CH];
#pragma unroll
          for (int j = 0; j < CH; j++) e[j] = (gk + j < k_ext) ? p[j] : (T)0;
          v = __builtin_bit_cast(u32x4, e);
        }
      } else {
        const T* p = ptr[i] + k0 * ld;
        if (gk < k_ext) {
          if (VEC) {
            if (mn_ok(i)) v = *reinterpret_cast<const u32x4*>(p);
          } else {
            const int64_t gmn = mn0 + mnofs(i);
            T e[CH];
#pragma unroll
            for (int j = 0; j < CH; j++) e[j] = (gmn + j < mn_ext) ? p[j] : (T)0;
            v = __builtin_bit_cast(u32x4, e);
          }
        }
      }
      regs[i] = v;
    }
  }

  // Writes the loaded chunks of K step k0 to gather_out (K-contiguous A).
  template <bool VEC>
  __device__ __forceinline__ void store_gather(int64_t k0, const u32x4 (&regs)[TS::kPer]) const {
    if constexpr (KMAJ) {
      constexpr int CH = TS::kCh;
#pragma unroll
      for (int i = 0; i < TS::kPer; i++) {
        const int64_t gk = k0 + kofs(i);
        if (!mn_ok(i)) continue;
        T* dst = gout + (mn0 + mnofs(i)) * k_ext + gk;
        if (VEC) {
          if (gk + CH <= k_ext) *reinterpret_cast<u32x4*>(dst) = regs[i];
        } else {
          const auto e = __builtin_bit_cast(typename VecOf<T, CH>::type, regs[i]);
#pragma unroll
          for (int j = 0; j < CH; j++)
            if (gk + j < k_ext) dst[j] = e[j];
        }
      }
    }
  }

  __device__ __forceinline__ void store(typename Elem<E>::T* lds, const u32x4 (&regs)[TS::kPer]) const {
#pragma unroll
    for (int i = 0; i < TS::kPer; i++) *reinterpret_cast<u32x4*>(lds + TS::lds_off(mnofs(i), kofs(i))) = regs[i];
  }
};

// 16 (mn) x (64 bytes of k) fragment at tile offsets (mn0, k0): lane l gets the
// 16 bytes of k starting at k0 + (l / 16) * 16 bytes, for row mn0 + l % 16.
template <int E, int R, bool KMAJ>
__device__ __forceinline__ u32x4 read_frag(const typename Elem<E>::T* lds, int mn0, int k0) {
  using TS = Tile<E, R, KMAJ>;
  const int l = threadIdx.x % 64;
  const int t = l % 16, g = l / 16;
  if constexpr (KMAJ) {
    return *reinterpret_cast<const u32x4*>(lds + (mn0 + t) * TS::kPitch + k0 + g * TS::kCh);
  } else if constexpr (E == 2) {
    const uint16_t* p0 = lds + (k0 + 8 * g + t / 4) * TS::kPitch + mn0 + 4 * (t % 4);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + 4 * TS::kPitch));
    const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(u32x4, v);
  } else {
    const uint8_t* p0 = lds + (k0 + 16 * g + t / 2) * TS::kPitch + mn0 + 8 * (t % 2);
    const i32x2 lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)p0);
    const i32x2 hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p0 + 8 * TS::kPitch));
    const u32x4 v = {(uint32_t)lo[0], (uint32_t)lo[1], (uint32_t)hi[0], (uint32_t)hi[1]};
    return v;
  }
}

// Problem description handed to the shared kernel.
struct Problem {
  const void* a_parts[kMaxRanks];
  int64_t rows_per_part;  // row block size of a gathered K-contiguous A
  const void* b;
  void* gather_out;       // optional copy of the gathered A
  int64_t m, n, k;
  int tile_order_cols;
};

// Choose the XCD-aware tile of workgroup blockIdx.x.
__device__ __forceinline__ void tile_of_block(int64_t m, int64_t n, int bm, int bn, int cols_order, int& tm, int& tn) {
  const int tiles_m = (int)((m + bm - 1) / bm), tiles_n = (int)((n + bn - 1) / bn);
  const int tiles = tiles_m * tiles_n;
  int lin = blockIdx.x;
  if (tiles % 8 == 0) lin = (blockIdx.x % 8) * (tiles / 8) + blockIdx.x / 8;
  if (cols_order) {
    tn = lin / tiles_m;
    tm = lin % tiles_m;
  } else {
    tm = lin / tiles_n;
    tn = lin % tiles_n;
  }
}

// Main loop: accumulates the (BM/2) x (BN/2) block of this wavefront into acc.
// Ops supplies: typedef Acc (f32x4 / i32x4); static Acc mfma(u32x4 a, u32x4 b, Acc c).
template <int E, int BM, int BN, bool AK, bool BKM, bool VEC, typename Ops>
__device__ __forceinline__ void mainloop(const Problem& p, int64_t m0, int64_t n0, bool write_gather,
                                         typename Elem<E>::T* lds,
                                         typename Ops::Acc (&acc)[BM / 32][BN / 32]) {
  using TA = Tile<E, BM, AK>;
  using TB = Tile<E, BN, BKM>;
  using T = typename Elem<E>::T;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int kStage = TA::kLds + TB::kLds;
  constexpr int BK = TA::kBK;
  constexpr int MK = 64 / E;  // K elements per MFMA

  Loader<E, BM, AK> la;
  Loader<E, BN, BKM> lb;
  la.init(p.a_parts, AK ? p.rows_per_part : p.m, AK ? p.k : p.m, p.m, p.k, m0, p.gather_out);
  lb.init(&p.b, p.n, BKM ? p.k : p.n, p.n, p.k, n0, nullptr);

  const int wave = threadIdx.x / 64;
  const int wm = wave / 2, wn = wave % 2;

  // Global loads run two K steps ahead of the MFMAs: register set s % 2 holds
  // step s between its load and its LDS write.  Step kt is computed from LDS
  // buffer kt % 2 while step kt + 1 waits in registers and step kt + 2 is in
  // flight; after the MFMAs, step kt + 1 is written to the other buffer and
  // one barrier closes the step.
  u32x4 ra[2][TA::kPer], rb[2][TB::kPer];
  const int nk = (int)((p.k + BK - 1) / BK);
  const bool gather = write_gather;

  auto compute = [&](const T* As, const T* Bs) {
#pragma unroll
    for (int kk = 0; kk < BK; kk += MK) {
      u32x4 fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; i++) fa[i] = read_frag<E, BM, AK>(As, wm * WM + 16 * i, kk);
#pragma unroll
      for (int j = 0; j < FN; j++) fb[j] = read_frag<E, BN, BKM>(Bs, wn * WN + 16 * j, kk);
#pragma unroll
      for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++) acc[i][j] = Ops::mfma(fa[i], fb[j], acc[i][j]);
    }
  };

  la.template load<VEC>(0, ra[0]);
  lb.template load<VEC>(0, rb[0]);
  if (nk > 1) {
    la.template load<VEC>(BK, ra[1]);
    lb.template load<VEC>(BK, rb[1]);
  }
  la.store(lds, ra[0]);
  lb.store(lds + TA::kLds, rb[0]);
  if (gather) la.template store_gather<VEC>(0, ra[0]);
  __syncthreads();

  // one K step; S is the register set of step kt (static so the sets stay in registers)
  auto step = [&](int kt, auto S_) {
    constexpr int S = decltype(S_)::value;
    const T* As = lds + S * kStage;
    if (kt + 2 < nk) {
      la.template load<VEC>((int64_t)(kt + 2) * BK, ra[S]);
      lb.template load<VEC>((int64_t)(kt + 2) * BK, rb[S]);
    }
    compute(As, As + TA::kLds);
    if (kt + 1 < nk) {
      T* nxt = lds + (S ^ 1) * kStage;
      la.store(nxt, ra[S ^ 1]);
      lb.store(nxt + TA::kLds, rb[S ^ 1]);
      if (gather) la.template store_gather<VEC>((int64_t)(kt + 1) * BK, ra[S ^ 1]);
    }
    __syncthreads();
  };
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, std::integral_constant<int, 0>());
    if (kt + 1 < nk) step(kt + 1, std::integral_constant<int, 1>());
  }
}

// LDS elements the kernel needs: two operand stages, or the 16-bit C tile.
template <int E, int BM, int BN, bool AK, bool BKM>
constexpr int lds_bytes() {
  constexpr int stages = 2 * (Tile<E, BM, AK>::kLds + Tile<E, BN, BKM>::kLds) * E;
  constexpr int ctile = BM * (BN + 8) * 2;
  return stages > ctile ? stages : ctile;
}

// Writes a wavefront's rounded 16-bit C fragments to the LDS C tile, then the
// whole workgroup stores the tile with 16-byte row-contiguous stores.
// cvt(i, j, r, row, col) returns the 16-bit output bits of element r of
// fragment (i, j) at tile coordinates (row, col).
template <int BM, int BN, bool VEC, typename Cvt>
__device__ __forceinline__ void store_c16(uint16_t* lds, uint16_t* C, int64_t m, int64_t n, int64_t m0, int64_t n0,
                                          Cvt cvt) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int kPitch = BN + 8;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int wm = wave / 2, wn = wave % 2;
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++) {
      const int col = wn * WN + 16 * j + lane % 16;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int row = wm * WM + 16 * i + 4 * (lane / 16) + r;
        lds[row * kPitch + col] = cvt(i, j, r, row, col);
      }
    }
  __syncthreads();
  constexpr int kRowChunks = BN / 8;
  for (int c = threadIdx.x; c < BM * kRowChunks; c += kThreads) {
    const int row = c / kRowChunks, col = (c % kRowChunks) * 8;
    const int64_t grow = m0 + row, gcol = n0 + col;
    if (grow >= m) continue;
    const uint16_t* src = lds + row * kPitch + col;
    if (VEC && gcol + 8 <= n) {
      *reinterpret_cast<u32x4*>(C + grow * n + gcol) = *reinterpret_cast<const u32x4*>(src);
    } else {
      for (int j = 0; j < 8; j++)
        if (gcol + j < n) C[grow * n + gcol + j] = src[j];
    }
  }
}

// Bytes the L2s fetch with a row-wise vs a column-wise tile order: each XCD
// streams the whole of the operand it does not share.
inline bool prefer_column_order(int64_t m, int64_t n, int64_t k, int e) {
  const double a = (double)m * (double)k * e, b = (double)n * (double)k * e;
  return 8.0 * a + b < a + 8.0 * b;
}

// Pick a tile shape: maximise (useful MFMA work / issued) x (CU fill over the
// waves of workgroups), with a small bonus for bigger tiles.
struct TileChoice { int bm, bn; };
inline int pick_tile(int64_t m, int64_t n, const TileChoice* cands, int count, int cus = 256) {
  double best = -1.0;
  int pick = count - 1;
  for (int i = 0; i < count; i++) {
    const int64_t tm = (m + cands[i].bm - 1) / cands[i].bm, tn = (n + cands[i].bn - 1) / cands[i].bn;
    const int64_t tiles = tm * tn;
    const int64_t waves = (tiles + cus - 1) / cus;
    const double useful = (double)m * (double)n / ((double)tiles * cands[i].bm * cands[i].bn);
    const double fill = (double)tiles / (double)(waves * cus);
    const double score = useful * fill * (1.0 + 0.02 * (cands[i].bm * cands[i].bn) / (128.0 * 128.0));
    if (score > best + 1e-9) {
      best = score;
      pick = i;
    }
  }
  return pick;
}

}  // namespace gemm
}  // namespace mc2
