/*
 * Seeded synthetic input generator shared by the oracle tests, the GPU parity
 * tests and the benchmark.  It produces tensors only: it holds none of the
 * arithmetic of the operators being checked.
 *
 * Stream definition (counter based, so any slice can be generated on its own):
 *   key(seed, tid) = mix64((seed << 32) ^ tid ^ 0xD1B54A32D192ED03)
 *   word(i)        = mix64(key + (i + 1) * 0x9E3779B97F4A7C15)
 * where mix64 is the SplitMix64 finaliser (Steele, Lea, Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014).
 *
 * Distributions, element i of a tensor:
 *   UNIFORM  a + (b - a) * u,  u = (word(i) >> 40) * 2^-24 in [0, 1), in fp64
 *   INT      a + (word(i) >> 32) mod (b - a + 1)          (integers a..b)
 *   NORMAL   Box-Muller on the pair p = i / 2:
 *              u1 = ((word(2p) >> 11) + 1) * 2^-53  in (0, 1]
 *              u2 =  (word(2p+1) >> 11)    * 2^-53  in [0, 1)
 *              z  = sqrt(-2 ln u1) * (i even ? cos : sin)(2 pi u2)
 *            value = a + b * z   (a = mean, b = standard deviation)
 * The fp64 value is rounded to fp32, then to the storage type with
 * round-to-nearest-even: fp16 and bf16 (IEEE overflow to infinity),
 * FLOAT8_E4M3FN with saturation to +-448 (OCP 8-bit FP), INT8 by plain
 * conversion of the integer value, FLOAT8_E8M0 stores the integer value v as
 * the biased exponent 127 + v (so the element means 2^v).
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

enum { G_F32 = 0, G_F16 = 1, G_BF16 = 2, G_I8 = 3, G_E4M3FN = 5, G_E8M0 = 7 };
enum { D_UNIFORM = 0, D_INT = 1, D_NORMAL = 2 };

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t word(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * 0x9E3779B97F4A7C15ULL);
}

static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static uint16_t f32_to_f16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7e00u;
  if (a >= 0x477ff000u) return sign | 0x7c00u; /* >= 65520 rounds to inf */
  if (a < 0x38800000u) {                       /* below 2^-14: subnormal */
    /* value = a_f * 2^24 units of 2^-24; round that to an integer */
    float af;
    memcpy(&af, &a, 4);
    float scaled = af * 16777216.0f; /* exact: power of two */
    float r = nearbyintf(scaled);
    return sign | (uint16_t)r;
  }
  uint32_t mant = a & 0x7fffffu;
  int32_t exp = (int32_t)(a >> 23) - 127 + 15;
  uint32_t h = ((uint32_t)exp << 10) | (mant >> 13);
  uint32_t rest = mant & 0x1fffu;
  if (rest > 0x1000u || (rest == 0x1000u && (h & 1u))) h += 1;
  return sign | (uint16_t)h;
}

/* OCP FLOAT8_E4M3FN, RNE, saturating to +-448. */
static uint8_t f32_to_e4m3fn_sat(float f) {
  uint8_t sign = signbit(f) ? 0x80 : 0x00;
  float a = fabsf(f);
  if (isnan(f)) return 0x7f;
  if (a >= 448.0f) return sign | 0x7e;
  if (a == 0.0f) return sign;
  /* a lies in [2^E, 2^(E+1)); below 2^-6 the spacing stays 2^-9 (subnormals) */
  int e;
  frexp((double)a, &e);
  int E = e - 1;
  if (E < -6) E = -6;
  double n = nearbyint((double)a / ldexp(1.0, E - 3)); /* 3 fraction bits, ties to even */
  if (n >= 16.0) {                                      /* rounded up into the next binade */
    E += 1;
    n = 8.0;
  }
  int code = (E == -6 && n < 8.0) ? (int)n : (((E + 7) << 3) | ((int)n - 8));
  if (code > 0x7e) code = 0x7e;
  return sign | (uint8_t)code;
}

static void store(int dtype, double v, void* out, int64_t i) {
  float f = (float)v;
  switch (dtype) {
    case G_F32: ((float*)out)[i] = f; break;
    case G_F16: ((uint16_t*)out)[i] = f32_to_f16_rne(f); break;
    case G_BF16: ((uint16_t*)out)[i] = f32_to_bf16_rne(f); break;
    case G_I8: ((int8_t*)out)[i] = (int8_t)(int)v; break;
    case G_E4M3FN: ((uint8_t*)out)[i] = f32_to_e4m3fn_sat(f); break;
    case G_E8M0: ((uint8_t*)out)[i] = (uint8_t)(127 + (int)v); break;
    default: break;
  }
}

/* Fill out[0..n) with elements [start, start + n) of tensor (seed, tid). */
int mc2gen_fill(uint64_t seed, uint64_t tid, int dist, double a, double b, int dtype,
                int64_t start, int64_t n, void* out) {
  const uint64_t key = mix64((seed << 32) ^ tid ^ 0xD1B54A32D192ED03ULL);
  if (dist < 0 || dist > 2) return -1;
  if (dtype != G_F32 && dtype != G_F16 && dtype != G_BF16 && dtype != G_I8 && dtype != G_E4M3FN &&
      dtype != G_E8M0)
    return -2;
  if (dist == D_INT && b < a) return -3;
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; j++) {
    const uint64_t i = (uint64_t)(start + j);
    double v;
    if (dist == D_UNIFORM) {
      double u = (double)(word(key, i) >> 40) * 0x1p-24;
      v = a + (b - a) * u;
    } else if (dist == D_INT) {
      uint64_t span = (uint64_t)(int64_t)(b - a) + 1;
      v = a + (double)((word(key, i) >> 32) % span);
    } else {
      uint64_t p = i / 2;
      double u1 = (double)((word(key, 2 * p) >> 11) + 1) * 0x1p-53;
      double u2 = (double)(word(key, 2 * p + 1) >> 11) * 0x1p-53;
      double r = sqrt(-2.0 * log(u1));
      double t = 6.283185307179586476925286766559 * u2;
      v = a + b * r * ((i & 1) ? sin(t) : cos(t));
    }
    store(dtype, v, out, j);
  }
  return 0;
}

/* Raw stream words, for determinism checks. */
void mc2gen_words(uint64_t seed, uint64_t tid, int64_t start, int64_t n, uint64_t* out) {
  const uint64_t key = mix64((seed << 32) ^ tid ^ 0xD1B54A32D192ED03ULL);
  for (int64_t j = 0; j < n; j++) out[j] = word(key, (uint64_t)(start + j));
}
