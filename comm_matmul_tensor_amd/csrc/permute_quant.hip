// K2: AlltoAll permute + smooth scale + per-token dynamic int8 quantisation
// (aclnnAlltoAllQuantMatmul page, "function" formulas: permutedOut =
// commOut.permute(1, 0, 2).view(BS/rankSize, rankSize*H), then
// Quant(permutedOut * x1Scale)).
//
// One workgroup per token t.  The permute is pure addressing: row t of P is
// the concatenation over ranks j of x1 row j*(bs/r) + t, so consecutive
// threads read consecutive 16-byte chunks of the r source rows (coalesced)
// and nothing is written for P unless the caller asks for it.  The token's
// values stay in registers between the two passes:
//   pass 1  y = P * smooth in fp32 (exact: two 8- or 11-bit significands),
//           absmax over the row (wavefront then workgroup reduction; max is
//           exact in any order)
//   s       = absmax / 127 (IEEE division)
//   pass 2  q = clamp(rint(y / s), -127, 127) with the result of the IEEE
//           division and round-half-to-even (computed as y * (1/s) with an
//           exact fallback near ties, see quant_fast); an all-zero row gives
//           s = 0 and q = 0.
// HBM traffic: 2 B read + 1 B written per element, plus the 4-byte scale.
#include "device.hpp"
#include "kernels.hpp"

namespace mc2 {
namespace {

constexpr int kThreads = 512;
constexpr int kMaxUnits = 5;  // 16-element units per thread: r*h <= 40960

template <int DT>
__device__ __forceinline__ float dec16(uint32_t bits) {
  if constexpr (DT == DT_BF16) return bf16_bits_to_f32(bits & 0xFFFFu);
  else return f16_bits_to_f32(bits & 0xFFFFu);
}

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
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

// Why y * (1 / s) may replace the IEEE quotient y / s: with inv = RN(1 / s),
// RN(y * inv) is within |y / s| (2^-23 + 2^-48) <= 1.6e-5 of y / s when
// |y / s| <= 127 (1 + 2^-23), and RN(y / s) is within 3.9e-6 of y / s, so
// both round to the same integer unless y * inv lies within 2e-5 of a
// half-integer.  The kernel flags every element within 3e-5 and redoes it
// with the division.

// Vector path: h % 16 == 0, so every 16-element unit of P lies inside one
// source row and is 32-byte aligned.  All of the token's loads are issued
// first; y = P * smooth stays in registers between the two passes.
//
// Pass 2 per element, with inv = 1/s:  qa = y * inv;  c = med3(qa, -127, 127);
// m = c + 1.5 * 2^23, which rounds c to an integer with ties to even and
// leaves that integer's two's-complement low byte in the low byte of m's bit
// pattern (|c| <= 127 < 2^22), so the int8 code is one byte of m.  If
// |qa - rint(c)| >= 0.5 - 3e-5 the element is near a half-integer and the
// wavefront recomputes its codes with the IEEE division (see quant_fast).
template <int DT>
__global__ __launch_bounds__(kThreads) void permute_quant_vec(QuantArgs a) {
  __shared__ float red[kThreads / 64];
  const int64_t t = blockIdx.x;
  const int64_t T = a.bs / a.r;
  const int64_t cols = (int64_t)a.r * a.h;
  const int units = (int)(cols / 16);
  const uint16_t* x1 = static_cast<const uint16_t*>(a.x1);
  const uint16_t* sm = static_cast<const uint16_t*>(a.smooth);

  u32x4 raw[kMaxUnits][2], smr[kMaxUnits][2];
#pragma unroll
  for (int v = 0; v < kMaxUnits; v++) {
    const int u = threadIdx.x + v * kThreads;
    const int e = (u < units ? u : 0) * 16;  // column in P (r * h <= 40960)
    const int hh = (int)a.h;
    const int j = e / hh, c = e - j * hh;      // source rank block and column
    const u32x4* src = reinterpret_cast<const u32x4*>(x1 + (((int64_t)j * T + t) * a.h + c));
    if (u < units) {
      raw[v][0] = src[0];
      raw[v][1] = src[1];
    }
  }
  if (sm) {
#pragma unroll
    for (int v = 0; v < kMaxUnits; v++) {
      const int u = threadIdx.x + v * kThreads;
      if (u < units) {
        const u32x4* sp = reinterpret_cast<const u32x4*>(sm + (int64_t)u * 16);
        smr[v][0] = sp[0];
        smr[v][1] = sp[1];
      }
    }
  }
  // y, element 2w+b of half hlf of unit v: y[v][hlf*8 + 2w + b]
  float y[kMaxUnits][16];
  float amax = 0.0f;
#pragma unroll
  for (int v = 0; v < kMaxUnits; v++) {
    const int u = threadIdx.x + v * kThreads;
    if (u < units) {
#pragma unroll
      for (int hlf = 0; hlf < 2; hlf++)
#pragma unroll
        for (int w = 0; w < 4; w++)
#pragma unroll
          for (int b = 0; b < 2; b++) {
            float yy = dec16<DT>(raw[v][hlf][w] >> (16 * b));
            if (sm) yy *= dec16<DT>(smr[v][hlf][w] >> (16 * b));
            y[v][hlf * 8 + 2 * w + b] = yy;
            amax = fmaxf(amax, __builtin_fabsf(yy));
          }
    }
  }
  amax = block_max(amax, red);
  const float s = amax / 127.0f;
  if (threadIdx.x == 0) a.s1[t] = s;
  // The error bound of quant_fast needs |y / s| <= 127 (1 + 2^-23), which holds
  // when s is a normal number; rows with a subnormal scale use the division.
  const float inv = 1.0f / s;
  const bool fast = s >= 1.17549435e-38f;  // uniform over the workgroup
  constexpr float kMagic = 12582912.0f;    // 1.5 * 2^23

#pragma unroll
  for (int v = 0; v < kMaxUnits; v++) {
    const int u = threadIdx.x + v * kThreads;
    if (u < units) {
      const int64_t e = (int64_t)u * 16;
      u32x4 qv = {0u, 0u, 0u, 0u};
      if (amax > 0.0f) {
        bool near = !fast;
        uint32_t mb[16];
#pragma unroll
        for (int i = 0; i < 16; i++) {
          const float qa = y[v][i] * inv;
          const float c = __builtin_amdgcn_fmed3f(qa, -127.0f, 127.0f);
          const float m = c + kMagic;
          near |= __builtin_fabsf(qa - (m - kMagic)) >= 0.49997f;
          mb[i] = __float_as_uint(m);
        }
        if (near) {  // rare: redo this unit with the IEEE division
#pragma unroll
          for (int i = 0; i < 16; i++) mb[i] = (uint32_t)quant1(y[v][i], s);
        }
#pragma unroll
        for (int w = 0; w < 4; w++)
          qv[w] = (mb[4 * w] & 0xFFu) | ((mb[4 * w + 1] & 0xFFu) << 8) | ((mb[4 * w + 2] & 0xFFu) << 16) |
                  (mb[4 * w + 3] << 24);
      }
      *reinterpret_cast<u32x4*>(a.q + t * cols + e) = qv;
      if (a.permuted) {  // optional copy of P: reload the unit rather than keep it in registers
        const int hh = (int)a.h;
        const int j = (int)e / hh, c = (int)e - j * hh;
        const u32x4* src = reinterpret_cast<const u32x4*>(x1 + (((int64_t)j * T + t) * a.h + c));
        u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.permuted) + t * cols + e);
        dst[0] = src[0];
        dst[1] = src[1];
      }
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

}  // namespace

hipError_t launch_permute_quant(const QuantArgs& a, hipStream_t s) {
  const int64_t T = a.bs / a.r;
  const int64_t cols = (int64_t)a.r * a.h;
  if (T < 1 || cols < 1 || cols > (int64_t)kMaxUnits * kThreads * 16) return hipErrorInvalidValue;
  const bool vec = a.h % 16 == 0;
  if (a.dtype == DT_BF16) {
    if (vec) permute_quant_vec<DT_BF16><<<(unsigned)T, kThreads, 0, s>>>(a);
    else permute_quant_scalar<DT_BF16><<<(unsigned)T, kThreads, 0, s>>>(a);
  } else if (a.dtype == DT_F16) {
    if (vec) permute_quant_vec<DT_F16><<<(unsigned)T, kThreads, 0, s>>>(a);
    else permute_quant_scalar<DT_F16><<<(unsigned)T, kThreads, 0, s>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mc2
