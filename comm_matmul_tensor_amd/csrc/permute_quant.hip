// K2: AlltoAll permute + smooth scale + per-token dynamic int8 quantisation
// (aclnnAlltoAllQuantMatmul page, "function" formulas: permutedOut =
// commOut.permute(1, 0, 2).view(BS/rankSize, rankSize*H), then
// Quant(permutedOut * x1Scale)).
//
// The permute is pure addressing: row t of P is the concatenation over ranks
// j of x1 row j*(bs/r) + t, so consecutive threads read consecutive 16-byte
// chunks of the r source rows (coalesced) and nothing is written for P
// unless the caller asks for it.  Two kernels: permute_quant_pipe, a
// persistent grid that walks the tokens with the next tokens' loads in
// flight (h % 8 == 0, no permuted copy: the usual case), and one workgroup
// per token otherwise.  A token's values stay in registers between the two
// passes:
//   pass 1  y = P * smooth in fp32 (exact: two 8- or 11-bit significands),
//           absmax over the row (wavefront then workgroup reduction; max is
//           exact in any order)
//   s       = absmax / 127 (IEEE division)
//   pass 2  q = clamp(rint(y / s), -127, 127) with the result of the IEEE
//           division and round-half-to-even (computed as rint(y (1/s) + 128)
//           - 128 with the division as the fallback near ties, see quant8); an
//           all-zero row gives s = 0 and q = 0.
// HBM traffic: 2 B read + 1 B written per element, plus the 4-byte scale.
#include "device.hpp"
#include "kernels.hpp"

namespace mc2 {
namespace {

constexpr int kThreads = 512;   // general path
constexpr int kVecThreads = 1024;
constexpr int kMaxUnits = 3;    // 16-element units per thread of the vector path: r*h <= 49152

template <int DT>
__device__ __forceinline__ float dec16(uint32_t bits) {
  if constexpr (DT == DT_BF16) return bf16_bits_to_f32(bits & 0xFFFFu);
  else return f16_bits_to_f32(bits & 0xFFFFu);
}

// Maximum over the wavefront's 64 lanes of a non-negative value, as a
// wave-uniform result: DPP steps within each row of 16 lanes (quad swaps,
// half-row and row mirrors), then row 0 / 2's lane 15 into rows 1 / 3 and
// lane 31 into rows 2 and 3, so lane 63 holds the maximum.  Lanes a DPP step
// does not write read 0, which leaves their maximum unchanged.  (The
// shuffle loop it replaces took six LDS round trips per token.)
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_max_step(float v) {
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, false)));
}
__device__ __forceinline__ float wave_max_nonneg(float v) {
  v = dpp_max_step<0xB1, 0xF>(v);   // quad_perm 1,0,3,2
  v = dpp_max_step<0x4E, 0xF>(v);   // quad_perm 2,3,0,1
  v = dpp_max_step<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_max_step<0x140, 0xF>(v);  // row_mirror
  v = dpp_max_step<0x142, 0xA>(v);  // row_bcast:15
  v = dpp_max_step<0x143, 0xC>(v);  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max_nonneg(v);
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; w++) m = fmaxf(m, red[w]);
  return m;
}

__device__ __forceinline__ int quant1(float y, float s) {
  float r = __builtin_rintf(y / s);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int)r;
}

// The codes of eight values y (|y| <= amax, s = amax / 127 > 0, inv = RN(1 / s))
// packed low element first, without a division where that is exact.
//
// rb = RN(y inv + 128) (one fma) lies within 1.9e-5 of RN(y / s) + 128: its
// own rounding is at most 2^-17 (rb < 256), inv's relative error 2^-24
// contributes at most |y / s| 2^-24 <= 7.6e-6 (|y / s| <= 127 (1 + 2^-24)),
// and RN(y / s) is within 3.8e-6 of y / s.  So where rb is more than 3e-5
// from a half-integer, rint(rb) = rint(RN(y / s)) + 128, an integer in
// [1, 255]: v_cvt_pk_u8_f32 converts it exactly into its byte of the packed
// word, and flipping bit 7 of each byte gives the two's-complement byte of
// rint(rb) - 128.  Elements within 3e-5 of a half-integer (ties included)
// take the IEEE division, each behind its own branch, so a wavefront runs a
// division only for an element that some lane needs (all eight where s is
// subnormal, fast = false, and the bound above does not hold).
__device__ __forceinline__ u32x2 quant8(const float (&y)[8], float inv, float s, bool fast) {
  constexpr float kNear = 0.49997f;
  uint32_t w[2] = {0u, 0u};
  float dmax = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; e++) {
    const float rb = __builtin_fmaf(y[e], inv, 128.0f);
    const float ri = __builtin_rintf(rb);
    dmax = fmaxf(dmax, __builtin_fabsf(rb - ri));
    w[e / 4] = __builtin_amdgcn_cvt_pk_u8_f32(ri, e % 4, w[e / 4]);
  }
  u32x2 q = {w[0] ^ 0x80808080u, w[1] ^ 0x80808080u};
  if (!fast || dmax >= kNear) {  // rare: the flagged elements again, with the division
    uint32_t mb[8];
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const float rb = __builtin_fmaf(y[e], inv, 128.0f);
      const float ri = __builtin_rintf(rb);
      if (!fast || __builtin_fabsf(rb - ri) >= kNear) mb[e] = (uint32_t)quant1(y[e], s);
      else mb[e] = (uint32_t)((int)ri - 128);  // ri in [1, 255] here
    }
#pragma unroll
    for (int k = 0; k < 2; k++)
      q[k] = (__builtin_amdgcn_perm(mb[4 * k + 3], mb[4 * k + 2], 0x0c0c0400u) << 16) |
             __builtin_amdgcn_perm(mb[4 * k + 1], mb[4 * k], 0x0c0c0400u);
  }
  return q;
}

// Vector path: h % 16 == 0, so every 16-element unit of P lies inside one
// source row and is 32-byte aligned.  1024 threads per token, each owning
// U units (U is the smallest count that covers the row, at most 3); all of
// the token's loads are issued first and y = P * smooth stays in registers
// between the two passes.
//
// Pass 2: quant8 on each half of a unit.
template <int DT, int U>
__global__ __launch_bounds__(kVecThreads, 2) void permute_quant_vec(QuantArgs a) {
  __shared__ float red[kVecThreads / 64];
  const int64_t t = blockIdx.x;
  const int64_t T = a.bs / a.r;
  const int64_t cols = (int64_t)a.r * a.h;
  const int units = (int)(cols / 16);
  const int hh = (int)a.h;
  const uint16_t* x1 = static_cast<const uint16_t*>(a.x1);
  const uint16_t* sm = static_cast<const uint16_t*>(a.smooth);

  // unit u of P is 16 elements of source row j T + t, column c
  u32x4 raw[U][2];
#pragma unroll
  for (int v = 0; v < U; v++) {
    const int u = threadIdx.x + v * kVecThreads;
    if (u < units) {
      const int e = u * 16, j = e / hh, c = e - j * hh;
      const u32x4* src = reinterpret_cast<const u32x4*>(x1 + ((int64_t)j * T + t) * a.h + c);
      raw[v][0] = src[0];
      raw[v][1] = src[1];
    }
  }
  if (a.permuted) {  // optional copy of P, straight from the registers (they die here)
#pragma unroll
    for (int v = 0; v < U; v++) {
      const int u = threadIdx.x + v * kVecThreads;
      if (u < units) {
        u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.permuted) + t * cols + (int64_t)u * 16);
        dst[0] = raw[v][0];
        dst[1] = raw[v][1];
      }
    }
  }
  float y[U][16];
  float amax = 0.0f;
#pragma unroll
  for (int v = 0; v < U; v++) {
    const int u = threadIdx.x + v * kVecThreads;
    if (u < units) {
      u32x4 smr[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
      if (sm) {
        const u32x4* sp = reinterpret_cast<const u32x4*>(sm + u * 16);
        smr[0] = sp[0];
        smr[1] = sp[1];
      }
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const uint32_t xw = raw[v][i / 8][(i % 8) / 2] >> (16 * (i & 1));
        float yy = dec16<DT>(xw);
        if (sm) yy *= dec16<DT>(smr[i / 8][(i % 8) / 2] >> (16 * (i & 1)));
        y[v][i] = yy;
        amax = fmaxf(amax, __builtin_fabsf(yy));
      }
    }
  }
  amax = wave_max_nonneg(amax);
  if (threadIdx.x % 64 == 0) red[threadIdx.x / 64] = amax;
  __syncthreads();
  amax = red[0];
#pragma unroll
  for (int w = 1; w < kVecThreads / 64; w++) amax = fmaxf(amax, red[w]);
  const float s = amax / 127.0f;
  if (threadIdx.x == 0) a.s1[t] = s;
  // The error bound of the fast path needs |y / s| <= 127 (1 + 2^-23), which
  // holds when s is a normal number; rows with a subnormal scale use the division.
  const float inv = 1.0f / s;
  const bool fast = s >= 1.17549435e-38f;  // uniform over the workgroup (see quant8)
#pragma unroll
  for (int v = 0; v < U; v++) {
    const int u = threadIdx.x + v * kVecThreads;
    if (u < units) {
      const int64_t e = (int64_t)u * 16;
      u32x4 qv = {0u, 0u, 0u, 0u};
      if (amax > 0.0f) {
#pragma unroll
        for (int hlf = 0; hlf < 2; hlf++) {
          float y8[8];
#pragma unroll
          for (int i = 0; i < 8; i++) y8[i] = y[v][8 * hlf + i];
          const u32x2 q2 = quant8(y8, inv, s, fast);
          qv[2 * hlf] = q2[0];
          qv[2 * hlf + 1] = q2[1];
        }
      }
      *reinterpret_cast<u32x4*>(a.q + t * cols + e) = qv;
    }
  }
}

// Pipelined path (h % 8 == 0, no permuted_out copy): a persistent grid, one
// 1024-thread workgroup per CU, walks the tokens t = b, b + G, ...  Thread x
// owns the 16-byte column chunks x, x + 1024, ... (C of them) of every
// token, so its smoothing factors are loaded once and stay in registers, and
// the loads of the next D - 1 tokens are in flight while the current token
// is reduced, quantised and stored (with one token per workgroup every
// workgroup loaded, then reduced, then stored, and the loads came in
// bursts).  y = P * smooth is recomputed from the raw values in the second
// pass instead of being kept.  One barrier per token: the per-wavefront
// maxima go to a slot of `red` that alternates between tokens.
//
// The loads are non-temporal buffer loads (x1 below 2 GiB): a 32-bit offset
// per chunk and the token's row offset as a scalar.  Every load is issued
// unconditionally -- chunks past the row's end re-load the last chunk
// (neither counted nor stored), and loads past the workgroup's last token
// re-load that token (an L2 hit) -- so no branch separates a load from its
// use and the compiler waits only for the token being processed.
constexpr int kPipeThreads = 1024;
constexpr int kMaxChunks = 5;    // 16-byte chunks per thread: r*h <= 5 * 8 * 1024 = 40960
// Cache policy of the x1 loads: non-temporal.  x1 is read exactly once, and
// streaming it past the caches keeps it from evicting the dirty lines other
// kernels left there (each such eviction is a write-back in the middle of
// this kernel): 40.0 -> 27.5 us after a 512 MB write, 23.0 -> 26.0 us warm.
constexpr int kLoadNT = 2;

// D: tokens whose loads are in flight per workgroup (3 for up to 3 chunks per
// thread, 2 above, where a third set of buffers would spill registers)
template <int DT, int C, bool FULL, int D = (C <= 3 ? 3 : 2)>
__global__ __launch_bounds__(kPipeThreads, 1) void permute_quant_pipe(QuantArgs a) {
  __shared__ float red[2][kPipeThreads / 64];
  const int64_t T = a.bs / a.r, h = a.h;
  const int64_t cols = (int64_t)a.r * h;
  const int chunks = (int)(cols / 8);
  const uint16_t* sm = static_cast<const uint16_t*>(a.smooth);
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.x1), (short)0, (int)(a.bs * h * 2), 0x00020000);
  // chunk i of this thread: P elements [8 ch, 8 ch + 8) = source row j T + t, columns [c, c + 8)
  uint32_t voff[C];
  u32x4 smr[C];
  bool valid[C];
  const uint32_t one2 = DT == DT_BF16 ? 0x3F803F80u : 0x3C003C00u;  // two 16-bit ones
#pragma unroll
  for (int i = 0; i < C; i++) {
    const int ch = (int)threadIdx.x + i * kPipeThreads;
    valid[i] = FULL || ch < chunks;
    const int64_t e = (int64_t)(valid[i] ? ch : chunks - 1) * 8, j = e / h, c = e - j * h;
    voff[i] = (uint32_t)((j * T * h + c) * 2);
    smr[i] = sm ? *reinterpret_cast<const u32x4*>(sm + e) : u32x4{one2, one2, one2, one2};
  }
  const int G = (int)gridDim.x;
  const int n_my = (int)((T - blockIdx.x + G - 1) / G);  // tokens of this workgroup, >= 1
  u32x4 buf[D][C];
  auto issue = [&](u32x4 (&b)[C], int k) {
    const int64_t t = blockIdx.x + (int64_t)(k < n_my ? k : n_my - 1) * G;
    const int soff = (int)(t * h * 2);
#pragma unroll
    for (int i = 0; i < C; i++)
      b[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)voff[i], soff, kLoadNT));
  };
  auto yval = [&](const u32x4& raw, const u32x4& s, int k) {
    float y = dec16<DT>(raw[k / 2] >> (16 * (k & 1)));
    return y * dec16<DT>(s[k / 2] >> (16 * (k & 1)));
  };
  auto process = [&](const u32x4 (&b)[C], int k) {
    const int64_t t = blockIdx.x + (int64_t)k * G;
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < C; i++) {
      float cm = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; e++) cm = fmaxf(cm, __builtin_fabsf(yval(b[i], smr[i], e)));
      amax = fmaxf(amax, valid[i] ? cm : 0.0f);
    }
    amax = wave_max_nonneg(amax);
    float* slot = red[k & 1];
    if (threadIdx.x % 64 == 0) slot[threadIdx.x / 64] = amax;
    __syncthreads();
    amax = slot[0];
#pragma unroll
    for (int w = 1; w < kPipeThreads / 64; w++) amax = fmaxf(amax, slot[w]);
    const float s = amax / 127.0f;
    if (threadIdx.x == 0) a.s1[t] = s;
    const float inv = 1.0f / s;
    const bool fast = s >= 1.17549435e-38f;  // see quant8
    const bool nonzero = amax > 0.0f;
#pragma unroll
    for (int i = 0; i < C; i++) {
      float y8[8];
#pragma unroll
      for (int e = 0; e < 8; e++) y8[e] = yval(b[i], smr[i], e);
      u32x2 qv = quant8(y8, inv, s, fast);
      if (!nonzero) qv = u32x2{0u, 0u};  // an all-zero token: s = 0, codes 0
      if (valid[i]) *reinterpret_cast<u32x2*>(a.q + t * cols + ((int64_t)threadIdx.x + i * kPipeThreads) * 8) = qv;
    }
  };
  // Token by token, as the loop issues them: interleaved (as the compiler
  // scheduled them without the barrier) they set the waits at the top of the
  // loop, shared with the steady state, to vmcnt(7), (5), (3), (1): pass 1 of
  // a token then waited for most of the next token's loads.
#pragma unroll
  for (int d = 0; d < D; d++) {
    issue(buf[d], d);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int k0 = 0;; k0 += D) {
#pragma unroll
    for (int d = 0; d < D; d++) {
      process(buf[d], k0 + d);
      issue(buf[d], k0 + d + D);
      if (k0 + d + 1 == n_my) return;
    }
  }
}

// General path (h not a multiple of 16): element by element, two passes
// over global memory.  Same arithmetic as the vector path.
template <int DT>
__global__ __launch_bounds__(kThreads) void permute_quant_scalar(QuantArgs a) {
  __shared__ float red[kThreads / 64];
  const int64_t t = blockIdx.x;
  const int64_t T = a.bs / a.r;
  const int64_t cols = (int64_t)a.r * a.h;
  const uint16_t* x1 = static_cast<const uint16_t*>(a.x1);
  const uint16_t* sm = static_cast<const uint16_t*>(a.smooth);
  auto load = [&](int64_t e) {
    const int64_t j = e / a.h, c = e - j * a.h;
    const uint16_t bits = x1[(j * T + t) * a.h + c];
    float y = dec16<DT>(bits);
    if (sm) y *= dec16<DT>(sm[e]);
    return y;
  };
  float amax = 0.0f;
  for (int64_t e = threadIdx.x; e < cols; e += kThreads) amax = fmaxf(amax, __builtin_fabsf(load(e)));
  amax = block_max(amax, red);
  const float s = amax / 127.0f;
  if (threadIdx.x == 0) a.s1[t] = s;
  for (int64_t e = threadIdx.x; e < cols; e += kThreads) {
    a.q[t * cols + e] = (int8_t)(amax > 0.0f ? quant1(load(e), s) : 0);
    if (a.permuted) {
      const int64_t j = e / a.h, c = e - j * a.h;
      static_cast<uint16_t*>(a.permuted)[t * cols + e] = x1[(j * T + t) * a.h + c];
    }
  }
}

template <int DT>
void launch_vec(const QuantArgs& a, int units_per_thread, hipStream_t s) {
  const unsigned grid = (unsigned)(a.bs / a.r);
  switch (units_per_thread) {
    case 1: permute_quant_vec<DT, 1><<<grid, kVecThreads, 0, s>>>(a); break;
    case 2: permute_quant_vec<DT, 2><<<grid, kVecThreads, 0, s>>>(a); break;
    default: permute_quant_vec<DT, kMaxUnits><<<grid, kVecThreads, 0, s>>>(a); break;
  }
}

template <int DT, int C>
void launch_pipe_c(const QuantArgs& a, bool full, unsigned grid, hipStream_t s) {
  if (full) permute_quant_pipe<DT, C, true><<<grid, kPipeThreads, 0, s>>>(a);
  else permute_quant_pipe<DT, C, false><<<grid, kPipeThreads, 0, s>>>(a);
}

template <int DT>
void launch_pipe(const QuantArgs& a, int chunks_per_thread, hipStream_t s) {
  const int64_t T = a.bs / a.r;
  const unsigned grid = (unsigned)(T < 256 ? T : 256);
  const bool full = (int64_t)a.r * a.h == (int64_t)chunks_per_thread * kPipeThreads * 8;
  switch (chunks_per_thread) {
    case 1: launch_pipe_c<DT, 1>(a, full, grid, s); break;
    case 2: launch_pipe_c<DT, 2>(a, full, grid, s); break;
    case 3: launch_pipe_c<DT, 3>(a, full, grid, s); break;
    case 4: launch_pipe_c<DT, 4>(a, full, grid, s); break;
    default: launch_pipe_c<DT, kMaxChunks>(a, full, grid, s); break;
  }
}

}  // namespace

hipError_t launch_permute_quant(const QuantArgs& a, hipStream_t s) {
  const int64_t T = a.bs / a.r;
  const int64_t cols = (int64_t)a.r * a.h;
  if (T < 1 || cols < 1) return hipErrorInvalidValue;
  // pipelined path for h % 8 == 0 without the permuted copy; above 4 chunks
  // per thread (r h > 32768) it would spill a few registers, so rows that
  // split into 16-element units take the one-token-per-workgroup path there
  const int cpt = (int)((cols / 8 + kPipeThreads - 1) / kPipeThreads);
  if (a.h % 8 == 0 && cpt <= kMaxChunks && (cpt <= 4 || a.h % 16 != 0) && !a.permuted &&
      a.bs * a.h * 2 < ((int64_t)1 << 31)) {
    if (a.dtype == DT_BF16) launch_pipe<DT_BF16>(a, cpt, s);
    else if (a.dtype == DT_F16) launch_pipe<DT_F16>(a, cpt, s);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  // vector path when rows split into whole 16-element units and fit 3 units per thread
  const bool vec = a.h % 16 == 0 && cols <= (int64_t)kMaxUnits * kVecThreads * 16;
  const int upt = (int)((cols / 16 + kVecThreads - 1) / kVecThreads);
  if (a.dtype == DT_BF16) {
    if (vec) launch_vec<DT_BF16>(a, upt, s);
    else permute_quant_scalar<DT_BF16><<<(unsigned)T, kThreads, 0, s>>>(a);
  } else if (a.dtype == DT_F16) {
    if (vec) launch_vec<DT_F16>(a, upt, s);
    else permute_quant_scalar<DT_F16><<<(unsigned)T, kThreads, 0, s>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mc2
