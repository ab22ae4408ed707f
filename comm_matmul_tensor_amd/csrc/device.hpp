// Device-side helpers shared by the libmc2 kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace mc2 {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// dtype codes, mirroring mc2_dtype (kept as plain ints for template use)
enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_I8 = 3, DT_I32 = 4, DT_E4M3FN = 5, DT_E5M2 = 6, DT_E8M0 = 7 };

// 16-byte store of output that no later step of this kernel reads:
// non-temporal, so the output streams to memory without displacing the
// operands' lines from the caches or making the caches write back other
// dirty lines first.
__device__ __forceinline__ void store_out16(void* dst, u32x4 v) {
  __builtin_nontemporal_store(v, static_cast<u32x4*>(dst));
}

// fp32 -> bf16 bits, round to nearest even (the gfx950 conversion is RNE).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}
// Two fp32 values -> two 16-bit values (lo in bits 0-15), round to nearest
// even; bf16 converts both with one packed conversion.
template <int DT>
__device__ __forceinline__ uint32_t pack2_16(float lo, float hi);

// fp32 -> fp16 bits, round to nearest even.
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;
  return __builtin_bit_cast(uint16_t, h);
}
template <>
__device__ __forceinline__ uint32_t pack2_16<DT_BF16>(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
template <>
__device__ __forceinline__ uint32_t pack2_16<DT_F16>(float lo, float hi) {
  return (uint32_t)f32_to_f16_bits(lo) | ((uint32_t)f32_to_f16_bits(hi) << 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// fp64 -> fp32 with round-to-odd: truncate toward zero, then set the last
// bit if anything was dropped.  Rounding this result to a format with at
// most 22 significand bits (bf16, fp16) with RNE gives the same bits as
// rounding the fp64 value directly (Boldo & Melquiond, "Emulation of FMA
// and correctly rounded sums: proved algorithms using rounding to odd",
// IEEE TC 2008).
__device__ __forceinline__ float f64_to_f32_round_odd(double d) {
  float f = (float)d;
  double back = (double)f;
  if (back != d && d == d) {
    uint32_t u = __float_as_uint(f);
    if (__builtin_fabs(back) > __builtin_fabs(d)) u -= 1;  // step toward zero
    f = __uint_as_float(u | 1u);
  }
  return f;
}

// OCP E8M0 scale code -> fp64 (2^(b - 127); 0xFF is NaN).
__device__ __forceinline__ double e8m0_to_f64(uint32_t b) {
  b &= 0xFFu;
  if (b == 0xFFu) return __builtin_nan("");
  return __longlong_as_double((long long)(b + (1023 - 127)) << 52);
}

}  // namespace mc2
