// K7: int4 -> int8 widening of the A16W4 / A4W4 operands
// (aclnnAlltoAllQuantMatmul page, "constraints": A16W4 needs N even, A4W4
// needs H and N even; read as two's-complement int4 codes, two per byte along
// the last dimension, value 2i in the low nibble of byte i).
//
// gfx950 has no int4 matrix instruction, so the codes are sign-extended to
// int8 in one streaming pass and the int8 GEMM (K3) runs on the result with
// its direct-to-LDS staging: the widened operand costs one extra write and
// read of its int8 size, against a GEMM whose staging would otherwise go
// through registers.  Up to two ranges (A and B of A4W4) in one launch.
//
// Widening is exact: every code maps to the int8 of the same value.  HBM
// traffic: 1 B read + 2 B written per packed byte.
#include "device.hpp"
#include "kernels.hpp"

namespace mc2 {
namespace {

constexpr int kWidenThreads = 256;
constexpr int kPer = 4;  // 16-byte packed chunks in flight per thread

// Four bytes holding one code each in their low nibble: bit 3 copied into
// the upper four bits (no carries: each byte's product is 0 or 0xF0).
__device__ __forceinline__ uint32_t sext4x4(uint32_t x) { return x | (((x >> 3) & 0x01010101u) * 0xF0u); }

// One packed word (codes 0..7) -> two int8 words (codes 0..3, 4..7): the low
// and high nibbles are separated, interleaved back into code order with byte
// permutes (v_perm_b32: selectors 0..3 pick bytes of the second source,
// 4..7 of the first) and sign-extended.
__device__ __forceinline__ u32x2 widen_word(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;  // codes 0,2,4,6 and 1,3,5,7
  return u32x2{sext4x4(__builtin_amdgcn_perm(hi, lo, 0x05010400u)), sext4x4(__builtin_amdgcn_perm(hi, lo, 0x07030602u))};
}

__device__ __forceinline__ int8_t code(uint32_t nib) { return (int8_t)(nib >= 8 ? (int)nib - 16 : (int)nib); }

__global__ __launch_bounds__(kWidenThreads) void widen_int4_kernel(WidenArgs a) {
  const int which = (int64_t)blockIdx.x < a.blocks0 ? 0 : 1;
  const int64_t b = which ? (int64_t)blockIdx.x - a.blocks0 : (int64_t)blockIdx.x;
  const uint8_t* src = a.src[which];
  int8_t* dst = a.dst[which];
  const int64_t nb = a.bytes[which], full = nb / 16;  // whole 16-byte chunks
  const int64_t c0 = b * (kPer * kWidenThreads) + threadIdx.x;
  if (full > 0) {
    // every lane loads (an index past the end reads the last chunk again) so
    // no load sits behind a per-lane branch
    u32x4 v[kPer];
#pragma unroll
    for (int j = 0; j < kPer; j++) {
      const int64_t c = c0 + (int64_t)j * kWidenThreads;
      v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + (c < full ? c : full - 1));
    }
#pragma unroll
    for (int j = 0; j < kPer; j++) {
      const int64_t c = c0 + (int64_t)j * kWidenThreads;
      if (c < full) {
        const u32x2 w0 = widen_word(v[j][0]), w1 = widen_word(v[j][1]);
        const u32x2 w2 = widen_word(v[j][2]), w3 = widen_word(v[j][3]);
        u32x4* d = reinterpret_cast<u32x4*>(dst) + 2 * c;
        d[0] = u32x4{w0[0], w0[1], w1[0], w1[1]};
        d[1] = u32x4{w2[0], w2[1], w3[0], w3[1]};
      }
    }
  }
  // the last nb % 16 bytes: the thread whose first chunk is the one after the whole ones
  if (c0 == full) {
    for (int64_t i = 16 * full; i < nb; i++) {
      const uint32_t w = src[i];
      dst[2 * i] = code(w & 15u);
      dst[2 * i + 1] = code(w >> 4);
    }
  }
}

int64_t blocks_for(int64_t bytes) {
  const int64_t per = (int64_t)kPer * kWidenThreads;
  return (bytes / 16 + per) / per;  // one more chunk index than whole chunks: the tail's thread
}

}  // namespace

hipError_t launch_widen_int4(const WidenArgs& a, hipStream_t s) {
  WidenArgs w = a;
  for (int i = 0; i < 2; i++) {
    if (w.bytes[i] < 0 || (w.bytes[i] > 0 && (!w.src[i] || !w.dst[i]))) return hipErrorInvalidValue;
    if ((reinterpret_cast<uintptr_t>(w.src[i]) | reinterpret_cast<uintptr_t>(w.dst[i])) % 16 != 0)
      return hipErrorInvalidValue;
  }
  const int64_t b0 = w.bytes[0] > 0 ? blocks_for(w.bytes[0]) : 0;
  const int64_t b1 = w.bytes[1] > 0 ? blocks_for(w.bytes[1]) : 0;
  if (b0 + b1 == 0) return hipSuccess;
  if (b0 + b1 > 0x7FFFFFFF) return hipErrorInvalidValue;
  w.blocks0 = b0;
  widen_int4_kernel<<<(unsigned)(b0 + b1), kWidenThreads, 0, s>>>(w);
  return hipGetLastError();
}

}  // namespace mc2
