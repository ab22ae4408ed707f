// Tiled MFMA GEMM shared by K1 (16-bit float) and K3 (int8) on gfx950.
//
// C (m, n) = A (m, k) @ B (k, n) with 1- or 2-byte elements.  A is either
// K-contiguous ((m, k) row-major, possibly gathered from up to 8 row blocks
// held in separate buffers) or M-contiguous (stored (k, m)); B is either
// K-contiguous (stored (n, k)) or N-contiguous ((k, n) row-major).
//
// Geometry, counted in bytes, is the same for both element sizes: a step of
// the main loop covers 128 bytes of K, an MFMA consumes 64 bytes of K
// (v_mfma_f32_16x16x32_{bf16,f16}: 32 elements; v_mfma_i32_16x16x64_i8: 64),
// and every LDS transfer and MFMA operand fragment is a 16-byte chunk.
//
// Workgroup: 256 threads = 4 wavefronts in a 2 x 2 grid; each wavefront owns a
// (BM/2) x (BN/2) block of C as 16 x 16 MFMA tiles.
//
// LDS layout.  A K-contiguous operand tile is stored K-major: one 128-byte
// row per m (or n) index, rows packed densely, the eight 16-byte chunks of
// row r permuted by XOR with r % 8; each MFMA fragment is one ds_read_b128
// per lane (16 lanes read 16 rows at the same logical chunk).  An
// MN-contiguous operand tile stays as it is in memory: one row of R
// elements per k, its 16-byte chunks XOR-swizzled by k (mn_swz); each
// fragment is two transpose reads (ds_read_b64_tr_b16 / _b8), so no
// operand needs a transpose pass.
//
// Staging.  Fast path (whole K steps, 16-byte aligned rows; tiles may cross
// the M / N edges, their loads clamped): both operands go global -> LDS with
// direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds), no registers and
// no ds_write, into a ring of three LDS stages (two for the 256 x 256 tile);
// the schedule is described at mainloop_fast.  Checked path (ragged K or
// unaligned rows): bounds-tested register loads with zero fill into the
// K-major layout (MN-contiguous operands transposed in registers with
// v_perm_b32), two stages, one barrier per step.
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
constexpr int kRowBytes = 128;  // K bytes per main-loop step = bytes per LDS tile row

typedef __attribute__((address_space(1))) const void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// Byte offset of logical 16-byte chunk c of row r in a swizzled tile.
__device__ __forceinline__ int swz(int r, int c) { return r * kRowBytes + ((c ^ (r & 7)) << 4); }

template <int E>
struct Elem;
template <>
struct Elem<2> { typedef uint16_t T; };
template <>
struct Elem<1> { typedef uint8_t T; };

// Problem description handed to the shared kernel.
struct Problem {
  const void* a_parts[kMaxRanks];
  int64_t rows_per_part;  // row block size of a gathered K-contiguous A
  const void* b;
  void* gather_out;       // optional copy of the gathered A
  int64_t m, n, k;
  // K-contiguous A, general form: element (row, kk) of A lies at
  //   a_parts[block of row] + (kk / kseg) kseg_stride + (row in block) a_ld + (kk % kseg) E
  // (kseg = k, kseg_stride = 0 for a plain matrix; kseg < k addresses an A
  // whose K is split into segments stored apart, as the AlltoAll permute
  // does).  a_part_bytes: bytes of one row block's buffer.
  int64_t a_ld, kseg, kseg_stride, a_part_bytes;
  int tile_order_cols;
  int tile_group;         // tile rows (columns with tile_order_cols) per group of the tile order
  // Reduce-scatter routing (rs_out == NULL: off): rows [rs_row0, rs_row0 +
  // rs_rows) of C, this rank's block, are stored to rs_out (row t of the
  // block to row t) instead of C.
  void* rs_out;
  int64_t rs_row0, rs_rows;
  // Optional bias (n values of the output's 16-bit type) added to every row
  // of C in the epilogue before the rounding (NULL: none).
  const void* bias;
  // Arrival emulation (ready == NULL: off).  A arrives in `arrived` (the
  // gathered matrix) in pieces: rows [g rows_chunk, (g+1) rows_chunk) x
  // columns [s slab_cols, (s+1) slab_cols) may be read once
  // ready[g * slabs + s] == ready_value.  rows_chunk is a multiple of the
  // tile height, so a tile waits on one flag per slab.  A workgroup whose
  // wait times out reads the rest of its rows from a_parts (the shards)
  // instead and counts itself in *fallbacks.  wait_ticks: the longest wait
  // for one piece, in ticks of the 100 MHz real-time counter.
  const unsigned* ready;
  unsigned ready_value;
  unsigned* fallbacks;
  uint64_t wait_ticks;
  const void* arrived;
  int64_t rows_chunk;
  int64_t slab_cols;
  int slabs;
  int first_row_tile;     // tile row handed out first (also without arrival; 0 by default)
};

// Row pointer of K-contiguous operand row `row` (row blocks of rows_per_part
// rows live in separate buffers; resolved once per thread, outside the K loop).
__device__ __forceinline__ const uint8_t* kmajor_row(const void* const* parts, int64_t rows_per_part,
                                                     int64_t ld_bytes, int64_t row) {
  int part = 0;
  int64_t local = row;
  while (local >= rows_per_part) {
    local -= rows_per_part;
    part++;
  }
  return static_cast<const uint8_t*>(parts[part]) + local * ld_bytes;
}

// Waits until *flag == value (raised by the copy kernel once its piece of A
// is visible device-wide) or `ticks` of the 100 MHz real-time counter pass;
// returns whether the piece arrived.  The flag lives in uncached memory, so every poll reads
// memory.  Every wavefront polls for itself (the 64 lanes' loads of one
// address are one request).
__device__ __forceinline__ bool wait_flag(const unsigned* flag, unsigned value, uint64_t ticks) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) == value) return true;
    if (__builtin_amdgcn_s_memrealtime() - t0 > ticks) return false;
    __builtin_amdgcn_s_sleep(4);
  }
}

// Arrival prologue of the checked path: waits for every slab of the tile's
// row chunk and returns the Problem its main loop reads (A from the arrived
// buffer, or from the shards after a time-out).
__device__ __forceinline__ Problem arrival_problem(const Problem& p, int64_t m0) {
  __shared__ int s_ok;
  if (threadIdx.x == 0) {
    const unsigned* f = p.ready + (m0 / p.rows_chunk) * p.slabs;
    bool ok = true;
    for (int sl = 0; ok && sl < p.slabs; sl++) ok = wait_flag(f + sl, p.ready_value, p.wait_ticks);
    if (!ok) __hip_atomic_fetch_add(p.fallbacks, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_ok = ok;
  }
  __syncthreads();
  __atomic_thread_fence(__ATOMIC_ACQUIRE);
  Problem q = p;
  if (s_ok) {
    for (int i = 0; i < kMaxRanks; i++) q.a_parts[i] = p.arrived;
    q.rows_per_part = p.m;
  }
  return q;
}

// ---------------------------------------------------------------- MN-contiguous operand, transposed in registers
// Thread t < kBlocks owns the square block kb = t % 8 (K chunk), nb = t / 8.
template <int E, int R>
struct TransLoader {
  static constexpr int CH = 16 / E;          // elements per chunk = block side
  static constexpr int kBlocks = 8 * (R / CH);
  static_assert(kBlocks <= kThreads, "tile too wide for one block per thread");
  using T = typename Elem<E>::T;
  const T* src;  // element (k = CH * kb, n = n0 + CH * nb) at k0 = 0
  int64_t ld;    // elements between consecutive k rows
  bool active;

  __device__ __forceinline__ void init(const void* base, int64_t ld_elems, int64_t n0) {
    const int t = threadIdx.x, kb = t % 8, nb = t / 8;
    active = t < kBlocks;
    ld = ld_elems;
    src = static_cast<const T*>(base) + (int64_t)(CH * kb) * ld + n0 + CH * (active ? nb : 0);
  }
  __device__ __forceinline__ void load(int64_t k0, u32x4 (&r)[CH]) const {
    if (active) {
#pragma unroll
      for (int j = 0; j < CH; j++) r[j] = *reinterpret_cast<const u32x4*>(src + (k0 + j) * ld);
    }
  }
  // Whether this wavefront issues the loads (some lane active); uniform.
  static __device__ __forceinline__ bool wave_loads() {
    return (__builtin_amdgcn_readfirstlane(threadIdx.x) & ~63) < kBlocks;
  }
  // Bounds-checked variant for edge tiles: rows k >= k_ext and columns >= n_ext read as zero.
  __device__ __forceinline__ void load_checked(int64_t k0, int64_t k_ext, int64_t n_ext, int64_t n0,
                                               u32x4 (&r)[CH]) const {
    const int t = threadIdx.x, kb = t % 8, nb = t / 8;
#pragma unroll
    for (int j = 0; j < CH; j++) {
      r[j] = u32x4{0u, 0u, 0u, 0u};
      const int64_t kk = k0 + CH * kb + j;
      if (!active || kk >= k_ext) continue;
      const int64_t nn = n0 + CH * nb;
      const T* p = src + (k0 + j) * ld;
      if (nn + CH <= n_ext && (ld % CH) == 0 && (n0 % CH) == 0) {
        r[j] = *reinterpret_cast<const u32x4*>(p);
      } else {
        T e[CH];
#pragma unroll
        for (int x = 0; x < CH; x++) e[x] = (nn + x < n_ext) ? p[x] : (T)0;
        r[j] = __builtin_bit_cast(u32x4, e);
      }
    }
  }
  // Transpose and write: output i is row n = CH * nb + (i ^ s), s = nb & 1.
  __device__ __forceinline__ void store(uint8_t* tile, const u32x4 (&r)[CH]) const {
    if (!active) return;
    const int t = threadIdx.x, kb = t % 8, nb = t / 8, s = nb & 1;
    if constexpr (E == 2) {
      // out dword d = element i' of r[2d] (low half) and of r[2d + 1] (high half);
      // both sit in dword i'/2 = i/2, half i' % 2.
      const uint32_t sel_even = s ? 0x07060302u : 0x05040100u;  // for i even (i' % 2 == s)
      const uint32_t sel_odd = s ? 0x05040100u : 0x07060302u;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const uint32_t sel = (i & 1) ? sel_odd : sel_even;
        u32x4 o;
#pragma unroll
        for (int d = 0; d < 4; d++) o[d] = __builtin_amdgcn_perm(r[2 * d + 1][i / 2], r[2 * d][i / 2], sel);
        const int row = CH * nb + (i ^ s);
        *reinterpret_cast<u32x4*>(tile + swz(row, kb)) = o;
      }
    } else {
      // out dword d = byte i' of r[4d], r[4d+1], r[4d+2], r[4d+3]; byte i' lives in
      // dword i'/4 = i/4 at position x = (i % 4) ^ s.
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const uint32_t x = (uint32_t)((i & 3) ^ s);
        const uint32_t sel = x | ((4 + x) << 8) | (x << 16) | ((4 + x) << 24);
        u32x4 o;
#pragma unroll
        for (int d = 0; d < 4; d++) {
          const uint32_t lo = __builtin_amdgcn_perm(r[4 * d + 1][i / 4], r[4 * d][i / 4], sel);
          const uint32_t hi = __builtin_amdgcn_perm(r[4 * d + 3][i / 4], r[4 * d + 2][i / 4], sel);
          o[d] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
        }
        const int row = CH * nb + (i ^ s);
        *reinterpret_cast<u32x4*>(tile + swz(row, kb)) = o;
      }
    }
  }
};

// ---------------------------------------------------------------- K-contiguous operand, checked register path
template <int E, int R>
struct RegLoaderK {
  static constexpr int kPer = R / 32;  // 16-byte chunks per thread (R rows x 8 chunks / 256)
  using T = typename Elem<E>::T;
  const uint8_t* row_ptr[kPer];
  int64_t k_ext, mn_ext, mn0;

  __device__ __forceinline__ static int row_of(int i) { return (threadIdx.x + i * kThreads) / 8; }
  __device__ __forceinline__ static int chunk_of(int i) { return (threadIdx.x + i * kThreads) % 8; }

  int64_t kseg = 0, kseg_stride = 0;  // K segments (kseg = 0: one segment)

  __device__ __forceinline__ void init(const void* const* parts, int64_t rows_per_part, int64_t ld_bytes,
                                       int64_t mn_ext_, int64_t k_ext_, int64_t mn0_) {
    k_ext = k_ext_;
    mn_ext = mn_ext_;
    mn0 = mn0_;
#pragma unroll
    for (int i = 0; i < kPer; i++) {
      const int64_t row = mn0 + row_of(i);
      row_ptr[i] = kmajor_row(parts, rows_per_part, ld_bytes, row < mn_ext ? row : 0);
    }
  }
  __device__ __forceinline__ void load(int64_t k0, u32x4 (&r)[kPer]) const {
    constexpr int CH = 16 / E;
#pragma unroll
    for (int i = 0; i < kPer; i++) {
      r[i] = u32x4{0u, 0u, 0u, 0u};
      if (mn0 + row_of(i) >= mn_ext) continue;
      const int64_t gk = k0 + CH * chunk_of(i);
      if (kseg > 0 && kseg < k_ext) {  // segmented K: element by element
        T e[CH];
#pragma unroll
        for (int x = 0; x < CH; x++) {
          const int64_t g = gk + x, sg = g / kseg;
          e[x] = g < k_ext ? *(reinterpret_cast<const T*>(row_ptr[i] + sg * kseg_stride) + (g - sg * kseg)) : (T)0;
        }
        r[i] = __builtin_bit_cast(u32x4, e);
        continue;
      }
      const T* p = reinterpret_cast<const T*>(row_ptr[i]) + gk;
      if (gk + CH <= k_ext && (k_ext % CH) == 0) {
        r[i] = *reinterpret_cast<const u32x4*>(p);
      } else {
        T e[CH];
#pragma unroll
        for (int x = 0; x < CH; x++) e[x] = (gk + x < k_ext) ? p[x] : (T)0;
        r[i] = __builtin_bit_cast(u32x4, e);
      }
    }
  }
  __device__ __forceinline__ void store(uint8_t* tile, const u32x4 (&r)[kPer]) const {
#pragma unroll
    for (int i = 0; i < kPer; i++) *reinterpret_cast<u32x4*>(tile + swz(row_of(i), chunk_of(i))) = r[i];
  }
};

// ---------------------------------------------------------------- compute
// 16 (mn) x 64-byte fragment: lane l gets logical chunk c0 + l / 16 of row mn0 + l % 16.
__device__ __forceinline__ u32x4 read_frag(const uint8_t* tile, int mn0, int c0) {
  const int l = threadIdx.x % 64;
  return *reinterpret_cast<const u32x4*>(tile + swz(mn0 + l % 16, c0 + l / 16));
}

template <int BM, int BN, typename Ops>
__device__ __forceinline__ void compute_step(const uint8_t* As, const uint8_t* Bs,
                                             typename Ops::Acc (&acc)[BM / 32][BN / 32]) {
  constexpr int WM = BM / 2, WN = BN / 2, FM = WM / 16, FN = WN / 16;
  const int wave = threadIdx.x / 64, wm = wave / 2, wn = wave % 2;
#pragma unroll
  for (int c0 = 0; c0 < 8; c0 += 4) {
    u32x4 fa[FM], fb[FN];
#pragma unroll
    for (int i = 0; i < FM; i++) fa[i] = read_frag(As, wm * WM + 16 * i, c0);
#pragma unroll
    for (int j = 0; j < FN; j++) fb[j] = read_frag(Bs, wn * WN + 16 * j, c0);
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
      for (int j = 0; j < FN; j++) acc[i][j] = Ops::mfma(fb[j], fa[i], acc[i][j]);  // C layout: stage_c16
  }
}

// Up to four 16-byte LDS reads (LDS byte addresses a[0..N)) and the wait for
// them, in one asm block.  For reads of a stage that an earlier barrier has
// ordered after its loads: the compiler, which cannot tell the targets of
// loads into LDS still in flight from these addresses, would otherwise wait
// for those loads first.
template <int N>
__device__ __forceinline__ void lds_read_b128_waited(u32x4* v, const uint32_t* a) {
  static_assert(N >= 1 && N <= 4, "one to four reads");
  if constexpr (N == 4) {
    asm volatile(
        "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
  } else if constexpr (N == 3) {
    asm volatile("ds_read_b128 %0, %3\n\tds_read_b128 %1, %4\n\tds_read_b128 %2, %5\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2])
                 : "v"(a[0]), "v"(a[1]), "v"(a[2])
                 : "memory");
  } else if constexpr (N == 2) {
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1])
                 : "v"(a[0]), "v"(a[1])
                 : "memory");
  } else {
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v[0]) : "v"(a[0]) : "memory");
  }
}

// Copies the A tile of the step held in LDS to gather_out (K-contiguous A).
// ASMRD: the whole-tile path reads the stage with lds_read_b128_waited.
template <int E, int BM, bool ASMRD = false>
__device__ __forceinline__ void copy_gather(const uint8_t* As, void* gout, int64_t m, int64_t k, int64_t m0,
                                            int64_t k0, int tid) {
  using T = typename Elem<E>::T;
  constexpr int CH = 16 / E;
  constexpr int NG = BM / 32;
  if (m0 + BM <= m && k0 + CH * 8 <= k && k % CH == 0) {
    // the tile's rows and this step's K range lie inside the matrix: all LDS
    // reads first, one wait, then the stores (no per-lane branches, which
    // made every chunk wait for its own read and for every earlier one)
    u32x4 v[NG];
    if constexpr (ASMRD) {
      uint32_t a[NG];
#pragma unroll
      for (int i = 0; i < NG; i++) {
        const int c = tid + i * kThreads;
        a[i] = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)(As + swz(c / 8, c % 8));
      }
#pragma unroll
      for (int i = 0; i < NG; i += 4) {  // groups of four, then the rest
        if (i + 4 <= NG) lds_read_b128_waited<4>(v + i, a + i);
        else if (NG - i == 3) lds_read_b128_waited<3>(v + i, a + i);
        else if (NG - i == 2) lds_read_b128_waited<2>(v + i, a + i);
        else lds_read_b128_waited<1>(v + i, a + i);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NG; i++) {
        const int c = tid + i * kThreads;
        v[i] = *reinterpret_cast<const u32x4*>(As + swz(c / 8, c % 8));
      }
    }
#pragma unroll
    for (int i = 0; i < NG; i++) {
      const int c = tid + i * kThreads;
      store_out16(static_cast<T*>(gout) + (m0 + c / 8) * k + k0 + CH * (c % 8), v[i]);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < NG; i++) {
    const int c = tid + i * kThreads, row = c / 8, chunk = c % 8;
    const int64_t grow = m0 + row, gk = k0 + CH * chunk;
    if (grow >= m || gk >= k) continue;
    const u32x4 v = *reinterpret_cast<const u32x4*>(As + swz(row, chunk));
    T* dst = static_cast<T*>(gout) + grow * k + gk;
    if (gk + CH <= k && (k % CH) == 0) {
      store_out16(dst, v);
    } else {
      T e[CH];
      __builtin_memcpy(e, &v, 16);
      for (int x = 0; x < CH; x++)
        if (gk + x < k) dst[x] = e[x];
    }
  }
}

// vmcnt-only wait (gfx9 encoding: vmcnt bits [3:0] and [15:14]; expcnt and
// lgkmcnt at their maxima, i.e. not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without a memory fence: this wavefront's LDS accesses are
// complete (lgkmcnt 0) and its global loads stay in flight.  (__syncthreads
// would also wait for every outstanding global load.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------- MN-contiguous LDS layout
// Row k of the tile holds R elements (R * E bytes) as 16-byte chunks; chunk c
// sits at position c ^ mn_swz(k).  The XOR spreads the rows that one
// ds_read_b64_tr_b16 / _b8 instruction touches over all 64 banks (each half
// wavefront hits every bank once), which gfx950 then serves without
// conflicts.
template <int E, int R>
__device__ __forceinline__ int mn_swz(int k) {
  static_assert((E == 2 && (R == 224 || R == 128 || R == 256)) || (E == 1 && (R == 224 || R == 128)),
                "no swizzle for this tile");
  // 128 or 256 16-bit columns: a k row is one or two full bank rows, so the
  // bank of a chunk depends only on its position mod 16 and the same XOR
  // spreads the 8 k rows x 2 chunks of a half-wavefront transpose read
  if constexpr (E == 2 && R == 224) return 2 * ((k >> 3) & 1);
  else if constexpr (E == 2) return 2 * ((k & 3) | (((k >> 3) & 1) << 2));
  else if constexpr (R == 224) return (k >> 4) & 1;
  else return ((k >> 1) & 3) | (((k >> 4) & 1) << 2);
}
template <int E, int R>
__device__ __forceinline__ int swz_mn(int k, int c) { return k * (R * E) + ((c ^ mn_swz<E, R>(k)) << 4); }

// ---------------------------------------------------------------- direct-to-LDS staging
// One operand tile per step (R rows x 128 bytes of K = 8R slots of 16 bytes).
// Thread t fills slots s = t + 256 i, i < R / 32, so instruction i of
// wavefront w writes the 1 KB block 256 i + 64 w + lane, in lane order as
// the LDS-destination loads require; the address of each lane is chosen so
// that the block holds the swizzled layout.  Rows (K-major) or chunks
// (MN-major) past the matrix edge are clamped to the last valid one: their
// products land only in C elements the epilogue does not store.
//
// The loads are buffer loads into LDS (buffer_load_dwordx4 ... lds): each
// instruction has a wave-uniform buffer resource (base and byte size of the
// operand, or of the row block holding that instruction's 8 rows), a fixed
// 32-bit per-lane offset and the step's offset as a scalar, so issuing one
// takes no vector arithmetic.  A load past the resource's size returns zeros
// instead of faulting.  Requirements, checked by the launcher: every
// operand (or row block) below 2 GiB, and gathered row blocks a multiple of
// 8 rows (the 8 rows of one instruction then never straddle two blocks).
constexpr int kBufferFlags = 0x00020000;  // dword 3 of a raw buffer resource on gfx9

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferFlags);
}

template <int E, int R, bool KMAJ>
struct DmaOperand {
  static constexpr int kN = R / 32;  // DMA instructions per thread and step
  __amdgpu_buffer_rsrc_t rsrc[kN];   // instruction i's operand (wave-uniform)
  uint32_t voff[kN];                 // this lane's byte offset at step 0
  uint32_t step_bytes;               // distance between consecutive steps
  int lds_wave;                      // 1024 x this wavefront's index (wave-uniform)

  // K-contiguous operand: row r of the tile is matrix row mn0 + r, found in
  // the row blocks `parts` (rows_per_part rows each, ld_bytes per row).
  // part_bytes: bytes of each row block's buffer (the resource size).
  // t: the thread's index among the kThreads threads that issue the loads.
  __device__ __forceinline__ void init_k(const void* const* parts, int64_t rows_per_part, int64_t ld_bytes,
                                         int64_t mn0, int64_t mn_ext, int64_t part_bytes, int t) {
    const int w = __builtin_amdgcn_readfirstlane(t / 64);
    lds_wave = 1024 * w;
#pragma unroll
    for (int i = 0; i < kN; i++) {
      const int s = t + kThreads * i, row = s / 8, c = (s % 8) ^ (row & 7);
      const int64_t r = mn0 + row < mn_ext ? mn0 + row : mn_ext - 1;
      // the instruction's 8 rows (32 i + 8 w ...) lie in one row block
      int64_t g0 = mn0 + 32 * i + 8 * w;
      g0 = g0 < mn_ext ? g0 : mn_ext - 1;
      // row block of those rows: none to find for a single block; otherwise a
      // 32-bit division (m is below 2^31)
      const int64_t part = rows_per_part >= mn_ext ? 0 : (int64_t)((uint32_t)g0 / (uint32_t)rows_per_part);
      rsrc[i] = make_rsrc(parts[part], part_bytes);
      voff[i] = (uint32_t)((r - part * rows_per_part) * ld_bytes + c * 16);
    }
    step_bytes = kRowBytes;
  }
  // MN-contiguous operand stored (k_ext, mn) with ld_bytes between k rows;
  // mn_ext is a multiple of the 16-byte chunk.
  __device__ __forceinline__ void init_mn(const void* base, int64_t ld_bytes, int64_t k_ext, int64_t mn0,
                                          int64_t mn_ext, int t) {
    constexpr int CH = 16 / E, kChunks = R * E / 16;
    lds_wave = 1024 * __builtin_amdgcn_readfirstlane(t / 64);
#pragma unroll
    for (int i = 0; i < kN; i++) {
      const int s = t + kThreads * i, k = s / kChunks, c = (s % kChunks) ^ mn_swz<E, R>(k);
      int64_t col = mn0 + (int64_t)c * CH;
      if (col + CH > mn_ext) col = mn_ext - CH;
      rsrc[i] = make_rsrc(base, k_ext * ld_bytes);
      voff[i] = (uint32_t)(k * ld_bytes + col * E);
    }
    step_bytes = (uint32_t)((kRowBytes / E) * ld_bytes);
  }
  __device__ __forceinline__ void issue(uint8_t* tile, int64_t off) const {
#pragma unroll
    for (int i = 0; i < kN; i++) issue_one(tile, off, i);
  }
  // Instruction i alone; off = the step's byte offset.
  __device__ __forceinline__ void issue_one(uint8_t* tile, int64_t off, int i) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc[i], (lptr_t)(tile + 4096 * i + lds_wave), 16, (int)voff[i], (int)off,
                                             0, 0);
  }
};

// Whether the buffer-load staging covers this problem: every operand, or
// gathered row block, below 2 GiB, and gathered row blocks of a multiple of
// 8 rows.
inline bool dma_buffers_ok(int64_t a_block_bytes, int64_t b_bytes, int num_parts, int64_t rows_per_part) {
  const int64_t lim = (int64_t)1 << 31;
  return a_block_bytes < lim && b_bytes < lim && (num_parts == 1 || rows_per_part % 8 == 0);
}

// ---------------------------------------------------------------- fragment reads
// NF fragments of 16 rows (m or n) starting at tile row row0, for the K
// half kk (64 bytes of K) of a step.  MFMA operand layout: lane l holds row
// l % 16 and the 16 bytes of K at 16 (l / 16).
//  - K-major tile: one ds_read_b128 per fragment.
//  - MN-major tile: two transpose reads.  Within each 16-lane group, lane t
//    of ds_read_b64_tr_b16 receives element t % 4 of the 8-byte pieces
//    addressed by lanes 4 j + t / 4 (j = 0..3), so lane s addresses k row
//    s / 4, columns 4 (s % 4) .. + 3, and lane t ends up with column t of 4
//    consecutive k rows; ds_read_b64_tr_b8 does the same for 8 rows of bytes
//    (lane s: row s / 2, bytes 8 (s % 2) .. + 7).
template <int E, int R, bool KMAJ, int NF>
struct FragReader {
  static constexpr int kOffs = KMAJ ? 2 : NF;
  int off[kOffs];

  __device__ __forceinline__ void init(int row0) {
    const int l = threadIdx.x % 64, g = l / 16, s = l % 16;
    if constexpr (KMAJ) {
      const int row = row0 + s;
#pragma unroll
      for (int kk = 0; kk < 2; kk++) off[kk] = swz(row, 4 * kk + g);
    } else if constexpr (E == 2) {
#pragma unroll
      for (int j = 0; j < NF; j++) {
        const int k = 8 * g + s / 4, col = row0 + 16 * j + 4 * (s % 4);
        off[j] = swz_mn<E, R>(k, col / 8) + (col % 8) * 2;
      }
    } else {
#pragma unroll
      for (int j = 0; j < NF; j++) {
        const int k = 16 * g + s / 2, col = row0 + 16 * j + 8 * (s % 2);
        off[j] = swz_mn<E, R>(k, col / 16) + col % 16;
      }
    }
  }
  // The swizzles depend only on bits of k that kk and the second read leave unchanged.
  __device__ __forceinline__ void read(const uint8_t* tile, int kk, u32x4 (&f)[NF]) const {
#pragma unroll
    for (int j = 0; j < NF; j++) f[j] = read_one(tile, kk, j);
  }
  // Fragment j alone (one LDS read for a K-major tile, two for an MN-major one).
  __device__ __forceinline__ u32x4 read_one(const uint8_t* tile, int kk, int j) const {
    constexpr int P = R * E;  // bytes per k row of an MN-major tile
    if constexpr (KMAJ) {
      return *reinterpret_cast<const u32x4*>(tile + off[kk] + 16 * kRowBytes * j);
    } else if constexpr (E == 2) {
      const uint8_t* q = tile + off[j] + 32 * kk * P;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)q);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(q + 4 * P));
      const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
      return u32x4{a[0], a[1], b[0], b[1]};
    } else {
      const uint8_t* q = tile + off[j] + 64 * kk * P;
      const i32x2 lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)q);
      const i32x2 hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(q + 8 * P));
      return u32x4{(uint32_t)lo[0], (uint32_t)lo[1], (uint32_t)hi[0], (uint32_t)hi[1]};
    }
  }
};

// First K step of the rotated walk of tile (tm, tn) over nk steps (the fast
// loops with ROTK, and dma_waves_loop).  int8 (the GEMM of AlltoAllQuantMatmul):
// one step per tile row.  16-bit (the fused AllGatherMatmul loops): two steps
// per tile row and six per tile column, the best of the patterns measured on
// the 8 x (512, 4096) @ (4096, 1792) workload (one step per row: 66 us, 2 + 6:
// 60-62 us; spreads of 4 per row or 10 per column ran slower than no rotation).
// Arrival mode does not rotate: it takes K in the order its pieces arrive.
template <int E>
__device__ __forceinline__ int rot_start(int64_t tm, int64_t tn, int nk) {
  return (int)((E == 1 ? tm : 2 * tm + 6 * tn) % nk);
}

// Fast path: k is a multiple of the step and every operand row is 16-byte
// aligned; tiles may cross the M / N edges (clamped loads).  Three LDS stages
// (separate arrays, so the compiler can tell a DMA target from the buffer
// being read) hold steps kt, kt+1, kt+2; the MFMA fragments of the two K
// halves of a step alternate between two register sets.  Step kt:
//   issue the DMA of step kt+2 (its stage was last read before the previous
//   barrier); read half 1 of step kt; MFMAs of half 0;
//   wait for the DMA of step kt+1, barrier;
//   read half 0 of step kt+1; MFMAs of half 1.
// The barrier sits between two blocks of MFMAs, and every LDS read has a
// block of MFMAs to hide behind.
//
// Arrival (ARR, K-contiguous A only): A is read from p.arrived, and the DMA
// of a step that starts a new slab of K is issued only once that slab of
// the tile's row chunk has arrived.  Each wavefront polls the flag of the
// slab two steps ahead just before issuing the DMA of the step after next,
// so the poll completes under the wait every step already makes and a slab
// that is on time costs no extra wait.  A wavefront whose wait times out
// reads the rest of A from the shards.
//
// Two stages (NS = 2, for tiles whose three stages would not fit in LDS):
// the DMA of step kt+2 goes into step kt's own stage during half 1 of step
// kt, right after the barrier that ends every read of that stage, and has
// until the barrier of step kt+1 to land (one step, against one and a half
// with three stages):
//   read half 1 of step kt; MFMAs of half 0;
//   wait for the DMA of step kt+1, barrier;
//   issue the DMA of step kt+2; read half 0 of step kt+1; MFMAs of half 1.
// TAG: distinguishes the specialisation the gather-wavefront kernel uses from
// the one run_mainloop uses (with one shared specialisation the compiler
// rejected the second use as a substitution failure).
//
// NODMA: another group of four wavefronts issues every DMA and waits for it
// before each barrier (dma_waves_loop); these wavefronts only read the
// stages, multiply and meet the barriers.
template <int E, int BM, int BN, bool AK, bool BKM, bool GATHER, bool ARR, int NS, typename Ops, int TAG = 0,
          bool NODMA = false, bool ROTK = false>
__device__ __forceinline__ void mainloop_fast(const Problem& p, int64_t m0, int64_t n0, int gather_phase,
                                              int gather_every, uint8_t* L0, uint8_t* L1, uint8_t* L2,
                                              typename Ops::Acc (&acc)[BM / 32][BN / 32]) {
  static_assert(!ARR || (AK && !GATHER), "arrival needs a K-contiguous A and no gather copy");
  static_assert(NS == 3 || (NS == 2 && !ARR), "two stages: no arrival wait");
  static_assert(!NODMA || (NS == 3 && !ARR && !GATHER), "loads from other wavefronts: three stages only");
  static_assert(!ROTK || !NODMA, "rotated K walk: the wavefronts that issue the loads rotate");
  const int tid = (int)threadIdx.x;
  constexpr int BK = kRowBytes / E;  // K elements per step
  constexpr int kATile = BM * kRowBytes;
  constexpr int WM = BM / 2, WN = BN / 2, FM = WM / 16, FN = WN / 16;
  using DA = DmaOperand<E, BM, AK>;
  using DB = DmaOperand<E, BN, BKM>;
  constexpr int ND = DA::kN + DB::kN;  // DMA instructions per thread and step
  DA da;
  DB db;
  DA da_shards;  // arrival: A from the shards, for a wavefront whose wait timed out
  if constexpr (ARR) {
    const void* arrived[1] = {p.arrived};
    da.init_k(arrived, p.m, p.k * E, m0, p.m, p.m * p.k * E, tid);
    da_shards.init_k(p.a_parts, p.rows_per_part, p.a_ld, m0, p.m, p.a_part_bytes, tid);
  } else if constexpr (NODMA) {
  } else if constexpr (AK) {
    da.init_k(p.a_parts, p.rows_per_part, p.a_ld, m0, p.m, p.a_part_bytes, tid);
  } else {
    da.init_mn(p.a_parts[0], p.m * E, p.k, m0, p.m, tid);
  }
  if constexpr (NODMA) {
  } else if constexpr (BKM) {
    const void* bparts[1] = {p.b};
    db.init_k(bparts, p.n, p.k * E, n0, p.n, p.n * p.k * E, tid);
  } else {
    db.init_mn(p.b, p.n * E, p.k, n0, p.n, tid);
  }
  const int wave = threadIdx.x / 64, wm = wave / 2, wn = wave % 2;
  FragReader<E, BM, AK, FM> ra;
  FragReader<E, BN, BKM, FN> rb;
  ra.init(wm * WM);
  rb.init(wn * WN);
  const int nk = (int)(p.k / BK);
  int next_gather = gather_phase;
  // ROTK: the workgroup walks K from step rot (rot_start) and wraps around,
  // so the workgroups that share a band of B (one per tile row) or of A (one
  // per tile column) read it a few steps apart instead of all at once.  Step
  // kt of the loop loads (and waits for, copies) physical step phys(kt); the
  // accumulation order follows, the same in every loop that rotates.
  const int rot = ROTK ? rot_start<E>(m0 / BM, n0 / BN, nk) : 0;
  auto phys = [&](int kt) {
    if constexpr (ROTK) return kt + rot >= nk ? kt + rot - nk : kt + rot;
    else return kt;
  };

  // arrival: the flags of this tile's row chunk, one per slab of K
  const unsigned* flags = ARR ? p.ready + (m0 / p.rows_chunk) * p.slabs : nullptr;
  const int sps = ARR ? (int)(p.slab_cols / BK) : 1;  // steps per slab
  bool fell_back = false;
  unsigned pv = 0;  // polled flag of the slab of the step after next
  auto poll = [&](int kt) {
    return __hip_atomic_load(flags + phys(kt) / sps, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  };
  // Blocking wait for the slab of step kt; after a time-out A comes from the shards.
  auto wait_step = [&](int kt) {
    if (fell_back) return;
    if (!wait_flag(flags + phys(kt) / sps, p.ready_value, p.wait_ticks)) {
      fell_back = true;
      da = da_shards;
      if (threadIdx.x % 64 == 0) __hip_atomic_fetch_add(p.fallbacks, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };

  // A's offset of the next step to be loaded: steps go through K segment by
  // segment (one segment, kseg = k, for a plain or an M-contiguous A)
  const int seg_steps = (int)(p.kseg / BK);
  int64_t a_next = 0, seg_base = 0;
  int seg_left = seg_steps;
  int a_phys = rot;
  if constexpr (ROTK) {
    seg_base = (int64_t)(rot / seg_steps) * p.kseg_stride;
    a_next = seg_base + (int64_t)(rot % seg_steps) * da.step_bytes;
    seg_left = seg_steps - rot % seg_steps;
  }
  auto advance_a = [&]() {
    if constexpr (ROTK) {
      if (++a_phys == nk) {  // past the last step: back to step 0
        a_phys = 0;
        seg_base = 0;
        a_next = 0;
        seg_left = seg_steps;
        return;
      }
    }
    if (--seg_left == 0) {
      seg_base += p.kseg_stride;
      a_next = seg_base;
      seg_left = seg_steps;
    } else {
      a_next += da.step_bytes;
    }
  };

  u32x4 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
  auto dma = [&](uint8_t* L, int kt) {
    if constexpr (!NODMA) {
      da.issue(L, a_next);
      db.issue(L + kATile, (int64_t)phys(kt) * db.step_bytes);
      advance_a();
    }
  };
  // One K half: the FM x FN MFMAs on (fa, fb), with DMA instructions
  // [d0, d1) of step kt_dma (when dma_on) and the FM + FN fragment reads of
  // half kk of stage rd (when rd_on) spread evenly between them, in an order
  // the scheduler keeps (sched_barrier after every slot).  With one wavefront
  // per SIMD a burst of loads backs up the load path and stalls the
  // wavefront's MFMA issue; a few loads and reads between consecutive MFMAs
  // keep the matrix pipe fed.
  auto half = [&](const u32x4(&fa)[FM], const u32x4(&fb)[FN], auto D0_, auto D1_, bool dma_on, uint8_t* L,
                  int kt_dma, bool rd_on, const uint8_t* rd, int kk, u32x4(&ra_out)[FM], u32x4(&rb_out)[FN]) {
    constexpr int D0 = decltype(D0_)::value, D1 = decltype(D1_)::value;
    constexpr int NM = FM * FN, NF = FM + FN, NDH = D1 - D0;
    constexpr int kTail = NM >= 2 * NF ? NM - 2 * NF < 8 ? NM - 2 * NF : 8 : 0;
    const int64_t offa = a_next, offb = (int64_t)phys(kt_dma) * db.step_bytes;
#pragma unroll
    for (int q = 0; q < NM; q++) {
      acc[q / FN][q % FN] = Ops::mfma(fb[q % FN], fa[q / FN], acc[q / FN][q % FN]);
      if constexpr (NDH > 0) {
#pragma unroll
        for (int d = 0; d < NDH; d++)
          if ((d * NM) / NDH == q && dma_on) {
            if (D0 + d < DA::kN) da.issue_one(L, offa, D0 + d);
            else db.issue_one(L + kATile, offb, D0 + d - DA::kN);
          }
      }
      // reads in the order the next half consumes them (its MFMAs run row i
      // by row i: A fragment 0 with B fragments 0..FN-1, then A fragments
      // 1..FM-1), spread over all but the last kTail slots so the last one
      // lands before the barrier
#pragma unroll
      for (int f = 0; f < NF; f++)
        if ((f * (NM - kTail)) / NF == q && rd_on) {
          if (f == 0) ra_out[0] = ra.read_one(rd, kk, 0);
          else if (f <= FN) rb_out[f - 1] = rb.read_one(rd + kATile, kk, f - 1);
          else ra_out[f - FN] = ra.read_one(rd, kk, f - FN);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using C0 = std::integral_constant<int, 0>;
  using CD = std::integral_constant<int, ND>;
  // FULL: steps kt+1 and kt+2 exist (no branches around the DMA and the reads).
  auto step = [&](int kt, auto FULL_, uint8_t* cur, uint8_t* nxt, uint8_t* nn) {
    constexpr bool FULL = decltype(FULL_)::value;
    const bool dma2 = FULL || kt + 2 < nk;
    // gather_out copy of this step's A tile (NG stores per thread, older than
    // every load issued below, so the wait below covers them)
    if (GATHER && kt == next_gather) {
      copy_gather<E, BM>(cur, p.gather_out, p.m, p.k, m0, (int64_t)phys(kt) * BK, (int)threadIdx.x);
      next_gather += gather_every;
    }
    if constexpr (ARR) {
      // the slab of step kt+2 (polled during the previous step) must have arrived
      if (dma2 && phys(kt + 2) % sps == 0 && pv != p.ready_value) wait_step(kt + 2);
      if (!fell_back && kt + 3 < nk && phys(kt + 3) % sps == 0) pv = poll(kt + 3);
    }
    __builtin_amdgcn_sched_barrier(0);
    // half 0 of step kt; the DMA of step kt+2 (its stage was last read
    // before the previous barrier); reads of half 1 of step kt
    half(fa0, fb0, C0(), CD(), dma2 && !NODMA, nn, kt + 2, true, cur, 1, fa1, fb1);
    if (dma2 && !NODMA) advance_a();
    // the DMA of step kt+1 (issued during step kt-1) has landed; only this
    // step's may still fly
    if constexpr (!NODMA) {
      if (dma2) wait_vmcnt<ND>();
      else wait_vmcnt<0>();
    }
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // half 1 of step kt; reads of half 0 of step kt+1
    half(fa1, fb1, C0(), C0(), false, nn, kt + 2, FULL || kt + 1 < nk, nxt, 0, fa0, fb0);
    __builtin_amdgcn_sched_barrier(0);
  };
  // Two stages.  FULL: steps kt+1 and kt+2 exist.
  auto step2 = [&](int kt, auto FULL_, uint8_t* cur, uint8_t* nxt) {
    constexpr bool FULL = decltype(FULL_)::value;
    const bool dma2 = FULL || kt + 2 < nk;
    if (GATHER && kt == next_gather) {
      copy_gather<E, BM>(cur, p.gather_out, p.m, p.k, m0, (int64_t)phys(kt) * BK, (int)threadIdx.x);
      next_gather += gather_every;
    }
    __builtin_amdgcn_sched_barrier(0);
    // half 0 of step kt; reads of half 1 of step kt
    half(fa0, fb0, C0(), C0(), false, cur, kt + 2, true, cur, 1, fa1, fb1);
    // the DMA of step kt+1 (issued during step kt-1) has landed
    wait_vmcnt<0>();
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // half 1 of step kt; the DMA of step kt+2 into this step's stage, which
    // no wavefront reads any more; reads of half 0 of step kt+1
    half(fa1, fb1, C0(), CD(), dma2, cur, kt + 2, FULL || kt + 1 < nk, nxt, 0, fa0, fb0);
    if (dma2) advance_a();
    __builtin_amdgcn_sched_barrier(0);
  };

  if constexpr (ARR) {
    wait_step(0);
    __atomic_thread_fence(__ATOMIC_ACQUIRE);  // no stale lines of A from earlier calls
    if (nk > 1 && phys(1) % sps == 0) wait_step(1);
    if (!fell_back && nk > 2 && phys(2) % sps == 0) pv = poll(2);
  }
  if constexpr (!NODMA) {
    dma(L0, 0);
    if (nk > 1) {
      dma(L1, 1);
      wait_vmcnt<ND>();
    } else {
      wait_vmcnt<0>();
    }
  }
  lds_barrier();
  ra.read(L0, 0, fa0);
  rb.read(L0 + kATile, 0, fb0);
  using Full = std::integral_constant<bool, true>;
  using Part = std::integral_constant<bool, false>;
  int kt = 0;
  if constexpr (NS == 2) {
    for (; kt + 3 < nk; kt += 2) {
      step2(kt, Full(), L0, L1);
      step2(kt + 1, Full(), L1, L0);
    }
    if (kt < nk) step2(kt, Part(), L0, L1);
    if (kt + 1 < nk) step2(kt + 1, Part(), L1, L0);
    if (kt + 2 < nk) step2(kt + 2, Part(), L0, L1);
  } else {
    for (; kt + 4 < nk; kt += 3) {
      step(kt, Full(), L0, L1, L2);
      step(kt + 1, Full(), L1, L2, L0);
      step(kt + 2, Full(), L2, L0, L1);
    }
    if (kt < nk) step(kt, Part(), L0, L1, L2);
    if (kt + 1 < nk) step(kt + 1, Part(), L1, L2, L0);
    if (kt + 2 < nk) step(kt + 2, Part(), L2, L0, L1);
    if (kt + 3 < nk) step(kt + 3, Part(), L0, L1, L2);
  }
}

// Checked path (edge tiles, ragged K): bounds-tested register
// loads into the same LDS layout, loads of step k+1 overlapping step k.
template <int E, int BM, int BN, bool AK, bool BKM, typename Ops>
__device__ __forceinline__ void mainloop_checked(const Problem& p, int64_t m0, int64_t n0, int gather_phase,
                                                 int gather_every, uint8_t* s0, uint8_t* s1,
                                                 typename Ops::Acc (&acc)[BM / 32][BN / 32]) {
  constexpr int BK = kRowBytes / E;
  constexpr int kATile = BM * kRowBytes;
  using LA = typename std::conditional<AK, RegLoaderK<E, BM>, TransLoader<E, BM>>::type;
  using LB = typename std::conditional<BKM, RegLoaderK<E, BN>, TransLoader<E, BN>>::type;
  constexpr int NA = AK ? BM / 32 : 16 / E;
  constexpr int NB = BKM ? BN / 32 : 16 / E;
  LA la;
  LB lb;
  if constexpr (AK) {
    la.init(p.a_parts, p.rows_per_part, p.a_ld, p.m, p.k, m0);
    la.kseg = p.kseg;
    la.kseg_stride = p.kseg_stride;
  } else {
    la.init(p.a_parts[0], p.m, m0);
  }
  const void* bparts[1] = {p.b};
  if constexpr (BKM) lb.init(bparts, p.n, p.k * E, p.n, p.k, n0);
  else lb.init(p.b, p.n, n0);
  auto loadA = [&](int64_t k0, u32x4 (&r)[NA]) {
    if constexpr (AK) la.load(k0, r);
    else la.load_checked(k0, p.k, p.m, m0, r);
  };
  auto loadB = [&](int64_t k0, u32x4 (&r)[NB]) {
    if constexpr (BKM) lb.load(k0, r);
    else lb.load_checked(k0, p.k, p.n, n0, r);
  };
  u32x4 ra[NA], rb[NB];
  const int nk = (int)((p.k + BK - 1) / BK);
  loadA(0, ra);
  loadB(0, rb);
  la.store(s0, ra);
  lb.store(s0 + kATile, rb);
  __syncthreads();
  for (int kt = 0; kt < nk; kt++) {
    uint8_t* cur = (kt & 1) ? s1 : s0;
    uint8_t* nxt = (kt & 1) ? s0 : s1;
    if (kt + 1 < nk) {
      loadA((int64_t)(kt + 1) * BK, ra);
      loadB((int64_t)(kt + 1) * BK, rb);
    }
    if (AK && gather_every > 0 && kt % gather_every == gather_phase)
      copy_gather<E, BM>(cur, p.gather_out, p.m, p.k, m0, (int64_t)kt * BK, (int)threadIdx.x);
    compute_step<BM, BN, Ops>(cur, cur + kATile, acc);
    if (kt + 1 < nk) {
      la.store(nxt, ra);
      lb.store(nxt + kATile, rb);
    }
    __syncthreads();
  }
}

// LDS bytes per stage: the two K-major operand tiles.
template <int BM, int BN>
constexpr int stage_bytes() { return (BM + BN) * kRowBytes; }

// Runs the main loop variant this workgroup needs.  gather: copy the gathered
// A to p.gather_out, spread over the workgroups of the row of tiles (the
// workgroup of column tile tn copies the steps kt with kt % tiles_n == tn).
// ARR: arrival emulation (see mainloop_fast; the checked path waits for the
// whole row chunk first).
// GMODE: 0 = no gather copy, 1 = gather copy (p.gather_out set), 2 = decided
// from p.gather_out at run time (the first two compile one fast loop only).
// ROTK: the fast loops walk K from a step set by the tile (rot_start, see
// mainloop_fast); the checked loop walks K in order.
template <int E, int BM, int BN, bool AK, bool BKM, bool VEC, bool ARR, int NS, typename Ops, int GMODE = 2,
          bool ROTK = false>
__device__ __forceinline__ void run_mainloop(const Problem& p, int64_t m0, int64_t n0, int tn, int tiles_n,
                                             uint8_t* L0, uint8_t* L1, uint8_t* L2,
                                             typename Ops::Acc (&acc)[BM / 32][BN / 32]) {
  constexpr int BK = kRowBytes / E;
  const int gather_every = (AK && !ARR && p.gather_out != nullptr) ? tiles_n : 0;
  if constexpr (VEC) {
    if (p.k % BK == 0 && p.kseg % BK == 0) {  // whole steps, each inside one K segment
      if constexpr (ARR) {
        mainloop_fast<E, BM, BN, AK, BKM, false, true, NS, Ops, 0, false, ROTK>(p, m0, n0, tn, 0, L0, L1, L2, acc);
      } else if constexpr (AK && NS == 3 && GMODE == 1) {
        mainloop_fast<E, BM, BN, AK, BKM, true, false, NS, Ops, 0, false, ROTK>(p, m0, n0, tn, gather_every, L0, L1,
                                                                                 L2, acc);
      } else if constexpr (AK && NS == 3 && GMODE == 2) {
        if (gather_every > 0)
          mainloop_fast<E, BM, BN, AK, BKM, true, false, NS, Ops, 0, false, ROTK>(p, m0, n0, tn, gather_every, L0,
                                                                                   L1, L2, acc);
        else mainloop_fast<E, BM, BN, AK, BKM, false, false, NS, Ops, 0, false, ROTK>(p, m0, n0, tn, gather_every, L0,
                                                                                  L1, L2, acc);
      } else {
        // no gather copy with two stages (the host picks no two-stage tile
        // when gather_out is set)
        mainloop_fast<E, BM, BN, AK, BKM, false, false, NS, Ops>(p, m0, n0, tn, gather_every, L0, L1, L2, acc);
      }
      return;
    }
  }
  if constexpr (ARR) {
    const Problem q = arrival_problem(p, m0);
    mainloop_checked<E, BM, BN, AK, BKM, Ops>(q, m0, n0, tn, 0, L0, L1, acc);
  } else {
    mainloop_checked<E, BM, BN, AK, BKM, Ops>(p, m0, n0, tn, gather_every, L0, L1, acc);
  }
}

// The three-stage fast loop without the gather copy or arrival wait, for
// callers that have checked its conditions (whole steps, one K segment per
// step, 16-byte aligned rows, buffers within the DMA limits).
template <int E, int BM, int BN, bool AK, bool BKM, typename Ops>
__device__ __forceinline__ void run_fast_loop(const Problem& p, int64_t m0, int64_t n0, uint8_t* L0, uint8_t* L1,
                                              uint8_t* L2, typename Ops::Acc (&acc)[BM / 32][BN / 32]) {
  mainloop_fast<E, BM, BN, AK, BKM, false, false, 3, Ops, 1>(p, m0, n0, 0, 0, L0, L1, L2, acc);
}

// The same loop with its loads issued by another group of four wavefronts
// (dma_waves_loop, run beside it in the same workgroup).
template <int E, int BM, int BN, bool AK, bool BKM, typename Ops>
__device__ __forceinline__ void run_loop_nodma(const Problem& p, int64_t m0, int64_t n0, uint8_t* L0, uint8_t* L1,
                                               uint8_t* L2, typename Ops::Acc (&acc)[BM / 32][BN / 32]) {
  mainloop_fast<E, BM, BN, AK, BKM, false, false, 3, Ops, 2, true>(p, m0, n0, 0, 0, L0, L1, L2, acc);
}

// The loads of the three-stage loop for a group of four wavefronts that run
// mainloop_fast<..., NODMA> (tid: thread index within this group), plus the
// gather_out copy (the steps kt with kt % tiles_n == tn).  It meets the same
// barriers: the prologue's (after the loads of step 0 have landed), then one
// per step kt, before which the loads of step kt + 1 have landed.  After the
// barrier of step kt - 1 (the prologue's for kt = 0) no wavefront reads step
// kt - 1's stage any more, so the loads of step kt + 2 go there; the copy
// reads step kt's stage, which holds it until the barrier of step kt + 1.
// Loads and stores leave vmcnt in the order issued, so the wait for step
// kt + 1 lets this step's loads (ND per thread) and copy stores (NG, each
// lane one per 16-byte chunk of a whole tile; a partial tile waits longer)
// stay in flight.
template <int E, int BM, int BN, bool BKM>
__device__ __forceinline__ void dma_waves_loop(const Problem& p, int64_t m0, int64_t n0, int tn, int tiles_n,
                                               uint8_t* L0, uint8_t* L1, uint8_t* L2, int tid) {
  constexpr int BK = kRowBytes / E;
  constexpr int kATile = BM * kRowBytes;
  using DA = DmaOperand<E, BM, true>;
  using DB = DmaOperand<E, BN, BKM>;
  constexpr int ND = DA::kN + DB::kN, NG = BM / 32;
  DA da;
  DB db;
  da.init_k(p.a_parts, p.rows_per_part, p.a_ld, m0, p.m, p.a_part_bytes, tid);
  if constexpr (BKM) {
    const void* bparts[1] = {p.b};
    db.init_k(bparts, p.n, p.k * E, n0, p.n, p.n * p.k * E, tid);
  } else {
    db.init_mn(p.b, p.n * E, p.k, n0, p.n, tid);
  }
  const int nk = (int)(p.k / BK);
  const bool whole = m0 + BM <= p.m;  // the copy's whole-tile path: NG stores per lane
  const bool copy = p.gather_out != nullptr;
  int next = tn;
  // K walked from step rot_start, as mainloop_fast does with ROTK
  const int rot = rot_start<E>(m0 / BM, n0 / BN, nk);
  auto phys = [&](int kt) { return kt + rot >= nk ? kt + rot - nk : kt + rot; };
  auto dma = [&](uint8_t* L, int kt) {
    da.issue(L, (int64_t)phys(kt) * da.step_bytes);
    db.issue(L + kATile, (int64_t)phys(kt) * db.step_bytes);
  };
  // cur: stage of step kt; nn: stage of step kt + 2
  auto step = [&](int kt, uint8_t* cur, uint8_t* nn) {
    const bool dma2 = kt + 2 < nk;
    if (dma2) dma(nn, kt + 2);
    const bool cp = copy && kt == next;
    if (cp) {
      copy_gather<E, BM, true>(cur, p.gather_out, p.m, p.k, m0, (int64_t)phys(kt) * BK, tid);
      next += tiles_n;
    }
    if (kt + 1 < nk) {
      if (dma2) {
        if (cp && whole) wait_vmcnt<ND + NG>();
        else wait_vmcnt<ND>();
      } else {
        if (cp && whole) wait_vmcnt<NG>();
        else wait_vmcnt<0>();
      }
    }
    lds_barrier();
  };
  dma(L0, 0);
  if (nk > 1) {
    dma(L1, 1);
    wait_vmcnt<ND>();
  } else {
    wait_vmcnt<0>();
  }
  lds_barrier();
  int kt = 0;
  for (; kt + 3 <= nk; kt += 3) {
    step(kt, L0, L2);
    step(kt + 1, L1, L0);
    step(kt + 2, L2, L1);
  }
  if (kt < nk) step(kt, L0, L2);
  if (kt + 1 < nk) step(kt + 1, L1, L0);
}

// Choose the XCD-aware tile of workgroup blockIdx.x.  Workgroup b runs on XCD
// b % 8, so b is first renumbered to lin such that each XCD owns a
// contiguous 1/8 of the tiles.  lin then walks the tiles in groups of
// kTileGroup tile rows, column by column inside a group (cols_order: groups
// of tile columns, row by row), so the tiles an XCD runs at once form a
// compact block and the band of the operand its group shares stays in that
// XCD's L2 while the other operand streams past once (choose_tile_group
// picks the group size).  first_row_tile rotates the row tiles so that tile
// row comes first.
__device__ __forceinline__ void tile_of_block(int64_t m, int64_t n, int bm, int bn, int cols_order, int group, int& tm,
                                              int& tn, int first_row_tile = 0) {
  const int tiles_m = (int)((m + bm - 1) / bm), tiles_n = (int)((n + bn - 1) / bn);
  const int tiles = tiles_m * tiles_n;
  int lin = blockIdx.x;
  if (tiles % 8 == 0) lin = (blockIdx.x % 8) * (tiles / 8) + blockIdx.x / 8;
  // major: the dimension grouped (rows, or columns with cols_order); minor: the other
  const int n_major = cols_order ? tiles_n : tiles_m, n_minor = cols_order ? tiles_m : tiles_n;
  const int per_group = group * n_minor;
  const int first = (lin / per_group) * group;
  const int gsize = n_major - first < group ? n_major - first : group;
  const int r = lin % per_group;
  const int major = first + r % gsize, minor = r / gsize;
  tm = cols_order ? minor : major;
  tn = cols_order ? major : minor;
  tm = (tm + first_row_tile) % tiles_m;
}

// Writes a wavefront's rounded 16-bit C fragments to an LDS copy of the C tile
// (rows [0, BM/2) in h0, rows [BM/2, BM) in h1) and waits for the whole
// workgroup.  The MFMAs take B's fragment as their first operand and A's as
// the second, so they compute C^T: element r of accumulator (i, j) of lane l
// is C at row 16 i + l % 16 and column 16 j + 4 (l / 16) + r of the
// wavefront's block, and each lane writes its four consecutive columns with
// one 8-byte LDS store.  val(i, j, r, row, col) returns the fp32 value of that
// element at tile coordinates (row, col); DT is the 16-bit output format
// (round to nearest even, two values per conversion).
template <int BM, int BN, int DT, typename Val>
__device__ __forceinline__ void stage_c16(uint16_t* h0, uint16_t* h1, Val val) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int kPitch = BN + 8;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int wm = wave / 2, wn = wave % 2;
  uint16_t* half = wm ? h1 : h0;
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++) {
      const int row = 16 * i + lane % 16;  // row inside the half
      const int col = wn * WN + 16 * j + 4 * (lane / 16);
      const int trow = wm * WM + row;
      const uint32_t w0 = pack2_16<DT>(val(i, j, 0, trow, col), val(i, j, 1, trow, col + 1));
      const uint32_t w1 = pack2_16<DT>(val(i, j, 2, trow, col + 2), val(i, j, 3, trow, col + 3));
      *reinterpret_cast<u32x2*>(half + row * kPitch + col) = u32x2{w0, w1};
    }
  __syncthreads();
}

// Row chunk c of the staged tile: 8 elements of tile row `row` from column `col`.
template <int BM, int BN>
__device__ __forceinline__ const uint16_t* staged_chunk(const uint16_t* h0, const uint16_t* h1, int row, int col) {
  constexpr int WM = BM / 2, kPitch = BN + 8;
  return (row < WM ? h0 + row * kPitch : h1 + (row - WM) * kPitch) + col;
}

// Stores the staged tile with 16-byte row-contiguous stores.  With
// unrolled set, a tile wholly inside C takes an unrolled loop without bounds
// tests, so its LDS reads are issued together instead of one wait per chunk
// (16 chunks at a time: the 256 x 256 tile has 32; not after the gather
// copy, where it measured slower); other tiles take the checked loop.
template <int BM, int BN, int NTH = kThreads>
constexpr bool unrolled_store() { return BM * (BN / 8) % NTH == 0 && BM * (BN / 8) / NTH <= 32; }

// NTH: the threads of the workgroup that share the stores.
template <int BM, int BN, bool VEC, int NTH = kThreads>
__device__ __forceinline__ void store_c16_tile(const uint16_t* h0, const uint16_t* h1, uint16_t* C, int64_t m,
                                               int64_t n, int64_t m0, int64_t n0, bool unrolled = true) {
  constexpr int kRowChunks = BN / 8;
  if constexpr (VEC && unrolled_store<BM, BN, NTH>()) {
    if (unrolled && m0 + BM <= m && n0 + BN <= n) {
#pragma unroll 16
      for (int it = 0; it < BM * kRowChunks / NTH; it++) {
        const int c = threadIdx.x + it * NTH, row = c / kRowChunks, col = (c % kRowChunks) * 8;
        store_out16(C + (m0 + row) * n + n0 + col, *reinterpret_cast<const u32x4*>(staged_chunk<BM, BN>(h0, h1, row, col)));
      }
      return;
    }
  }
  for (int c = threadIdx.x; c < BM * kRowChunks; c += NTH) {
    const int row = c / kRowChunks, col = (c % kRowChunks) * 8;
    const int64_t grow = m0 + row, gcol = n0 + col;
    if (grow >= m) continue;
    const uint16_t* src = staged_chunk<BM, BN>(h0, h1, row, col);
    if (VEC && gcol + 8 <= n) {
      store_out16(C + grow * n + gcol, *reinterpret_cast<const u32x4*>(src));
    } else {
      for (int j = 0; j < 8; j++)
        if (gcol + j < n) C[grow * n + gcol + j] = src[j];
    }
  }
}

template <int BM, int BN, bool VEC, int DT, typename Val>
__device__ __forceinline__ void store_c16(uint16_t* h0, uint16_t* h1, uint16_t* C, int64_t m, int64_t n, int64_t m0,
                                          int64_t n0, Val val) {
  stage_c16<BM, BN, DT>(h0, h1, val);
  store_c16_tile<BM, BN, VEC>(h0, h1, C, m, n, m0, n0);
}

// LDS stages of the main loop: three, or two for the 256 x 256 tile (whose
// three stages would exceed the 160 KB of LDS).
template <int BM, int BN>
constexpr int lds_stages() { return BM * BN >= 256 * 256 ? 2 : 3; }

// LDS bytes of one stage array: an operand stage, or half of the 16-bit C tile.
template <int BM, int BN>
constexpr int lds_stage_array_bytes() {
  constexpr int st = stage_bytes<BM, BN>();
  constexpr int half_c = (BM / 2) * (BN + 8) * 2;
  return st > half_c ? st : half_c;
}

// Bytes the L2s fetch with a row-wise vs a column-wise tile order: each XCD
// streams the whole of the operand it does not share.
inline bool prefer_column_order(int64_t m, int64_t n, int64_t k, int e) {
  const double a = (double)m * (double)k * e, b = (double)n * (double)k * e;
  return 8.0 * a + b < a + 8.0 * b;
}

// Group size of the tile order: the 32 workgroups an XCD runs at once cover
// G tile rows x 32/G tile columns (transposed with cols_order), whose A and
// B bands its L2 must hold; pick the G with the smallest bands.
inline int choose_tile_group(int64_t m, int64_t n, int bm, int bn, int cols_order) {
  constexpr int kPerXcd = 32;
  const int64_t tiles_m = (m + bm - 1) / bm, tiles_n = (n + bn - 1) / bn;
  const int64_t major = cols_order ? tiles_n : tiles_m, minor = cols_order ? tiles_m : tiles_n;
  const int64_t wmaj = cols_order ? bn : bm, wmin = cols_order ? bm : bn;
  int best = 1;
  int64_t best_cost = -1;
  for (int64_t g = 1; g <= major && g <= kPerXcd; g++) {
    const int64_t cols = (kPerXcd + g - 1) / g;
    if (cols > minor && g < major) continue;
    const int64_t cost = g * wmaj + (cols < minor ? cols : minor) * wmin;
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = (int)g;
    }
  }
  return best;
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
