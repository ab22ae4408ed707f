// K4: QuantAllReduce dequantise-then-sum (QuantAllReduce README, "function"
// formula output = Reduce(AllGather(scales) * AllGather(x)) with sum).
//
// One pass streams the r ranks' low-bit shards and their scales from HBM and
// writes the sum once.  Each thread owns 16 consecutive elements of a row:
// one 16-byte load per rank (int8 / fp8 codes), one scale per rank (the 16
// elements lie inside one 128-element group, or one 32-element mx block),
// and two 16-byte vector stores (bf16 / fp16) or, for fp32, four 16-byte
// stores of consecutive wavefront output after an exchange through LDS.
//
// Arithmetic: every product code * scale is exact in fp64 (an int8 or fp8
// code has at most 8 significant bits, a scale 24 or 1), so the fp64 FMA
// chain over ranks 0..r-1 performs exactly the additions of the definition
// in rank order, and the result is rounded once: fp32 directly, bf16 / fp16
// through fp32 round-to-odd.
#include "device.hpp"
#include "kernels.hpp"

namespace mc2 {

namespace {

template <int XFMT, int BYTE>
__device__ __forceinline__ double decode_x(uint32_t word) {
  if constexpr (XFMT == DT_I8) {
    return (double)(int)(int8_t)((word >> (8 * BYTE)) & 0xFFu);
  } else if constexpr (XFMT == DT_E4M3FN) {
    return (double)__builtin_amdgcn_cvt_f32_fp8((int)word, BYTE);
  } else {
    return (double)__builtin_amdgcn_cvt_f32_bf8((int)word, BYTE);
  }
}

// acc[4w + j] += decode(byte j of word) * s for one 32-bit word of codes.
template <int XFMT>
__device__ __forceinline__ void fma_word(uint32_t word, double s, double* acc) {
  acc[0] = __builtin_fma(decode_x<XFMT, 0>(word), s, acc[0]);
  acc[1] = __builtin_fma(decode_x<XFMT, 1>(word), s, acc[1]);
  acc[2] = __builtin_fma(decode_x<XFMT, 2>(word), s, acc[2]);
  acc[3] = __builtin_fma(decode_x<XFMT, 3>(word), s, acc[3]);
}

template <int R, int XFMT, int SFMT, int OFMT>
__global__ __launch_bounds__(256) void dequant_sum_kernel(QarArgs a) {
  // fp32 output: each thread's 64 bytes are exchanged within the wavefront
  // through LDS so that every store instruction writes 1 KB of consecutive
  // output (whole 128-byte lines), streamed out with non-temporal stores.
  // Against four 16-byte stores per thread 64 bytes apart (plain stores):
  // QuantAllReduce int8 127.4 -> 120 us and QuantReduceScatter 24.4 -> 21 us in
  // the benchmark step, and the rows after it no longer find the cache full
  // of its dirty output (the AllGatherMatmul after it: 77.7 -> 74-75 us).
  // Plain coalesced stores made the int8 row faster (112 us) and the rows
  // after it slower; 16-bit output keeps its two 16-byte stores per thread
  // (exchanged, it measured 106-111 against 101-107 us).
  constexpr bool XCHG = OFMT == DT_F32;
  __shared__ u32x4 stage[XCHG ? 256 * 4 : 1];
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t e0 = g * 16;
  const bool active = e0 < a.total;
  if (!XCHG && !active) return;
  const int64_t ee = active ? e0 : 0;  // lanes past the end (exchange only) read element 0
  const int64_t t = ee / a.h;
  const int64_t c = ee - t * a.h;

  u32x4 xv[R];
#pragma unroll
  for (int i = 0; i < R; i++)  // streamed once: non-temporal loads
    xv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(a.x[i]) + ee));

  double sc[R];
#pragma unroll
  for (int i = 0; i < R; i++) {
    if constexpr (SFMT == DT_F32) {
      sc[i] = (double)static_cast<const float*>(a.scales[i])[t * (a.h >> 7) + (c >> 7)];
    } else {
      sc[i] = e8m0_to_f64(static_cast<const uint8_t*>(a.scales[i])[t * (a.h >> 5) + (c >> 5)]);
    }
  }

  double acc[16];
#pragma unroll
  for (int j = 0; j < 16; j++) acc[j] = 0.0;
#pragma unroll
  for (int i = 0; i < R; i++) {
#pragma unroll
    for (int w = 0; w < 4; w++) fma_word<XFMT>(xv[i][w], sc[i], acc + 4 * w);
  }

  if constexpr (XCHG) {
    // lane L keeps its 4 chunks at 16 (4 L + (v ^ ((L >> 2) & 3))) bytes of
    // the wavefront's 4 KB (the XOR puts lanes 4 apart on other banks); store
    // v of lane L then writes chunk 64 v + L of the wavefront's output
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
    u32x4* ws = stage + wave * 256;
#pragma unroll
    for (int v = 0; v < 4; v++) {
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; j++) w[j] = __builtin_bit_cast(uint32_t, (float)acc[4 * v + j]);
      ws[4 * lane + (v ^ ((lane >> 2) & 3))] = w;
    }
    __builtin_amdgcn_wave_barrier();
    const int64_t wbase = ((int64_t)blockIdx.x * 256 + wave * 64) * 16;  // the wavefront's first element
#pragma unroll
    for (int v = 0; v < 4; v++) {
      const int q = 64 * v + lane, tl = q / 4, j = q % 4;
      const u32x4 w = ws[4 * tl + (j ^ ((tl >> 2) & 3))];
      const int64_t e = wbase + 4 * (int64_t)q;  // whole chunks: total is a multiple of 16
      if (e < a.total) __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(static_cast<float*>(a.out) + e));
    }
  } else {
    uint16_t* o = static_cast<uint16_t*>(a.out) + e0;
#pragma unroll
    for (int v = 0; v < 2; v++) {
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const float lo = f64_to_f32_round_odd(acc[8 * v + 2 * j]);
        const float hi = f64_to_f32_round_odd(acc[8 * v + 2 * j + 1]);
        const uint32_t l = OFMT == DT_BF16 ? f32_to_bf16_bits(lo) : f32_to_f16_bits(lo);
        const uint32_t h = OFMT == DT_BF16 ? f32_to_bf16_bits(hi) : f32_to_f16_bits(hi);
        w[j] = l | (h << 16);
      }
      reinterpret_cast<u32x4*>(o)[v] = w;
    }
  }
}

template <int R, int XFMT, int SFMT>
hipError_t launch_o(const QarArgs& a, hipStream_t s) {
  const int64_t threads = a.total / 16;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  switch (a.out_dtype) {
    case DT_F32: dequant_sum_kernel<R, XFMT, SFMT, DT_F32><<<blocks, 256, 0, s>>>(a); break;
    case DT_BF16: dequant_sum_kernel<R, XFMT, SFMT, DT_BF16><<<blocks, 256, 0, s>>>(a); break;
    case DT_F16: dequant_sum_kernel<R, XFMT, SFMT, DT_F16><<<blocks, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int R>
hipError_t launch_r(const QarArgs& a, hipStream_t s) {
  if (a.scale_dtype == DT_F32) {
    if (a.x_dtype == DT_I8) return launch_o<R, DT_I8, DT_F32>(a, s);
    if (a.x_dtype == DT_E4M3FN) return launch_o<R, DT_E4M3FN, DT_F32>(a, s);
    if (a.x_dtype == DT_E5M2) return launch_o<R, DT_E5M2, DT_F32>(a, s);
  } else if (a.scale_dtype == DT_E8M0) {
    if (a.x_dtype == DT_E4M3FN) return launch_o<R, DT_E4M3FN, DT_E8M0>(a, s);
    if (a.x_dtype == DT_E5M2) return launch_o<R, DT_E5M2, DT_E8M0>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_dequant_sum(const QarArgs& a, hipStream_t s) {
  // h is a multiple of 128, so rows hold whole 16-element chunks
  if (a.total % 16 != 0 || a.h % 128 != 0) return hipErrorInvalidValue;
  switch (a.r) {
    case 2: return launch_r<2>(a, s);
    case 4: return launch_r<4>(a, s);
    case 8: return launch_r<8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mc2
