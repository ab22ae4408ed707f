/*
 * mc2_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU implementation of what the MC2
 * per-rank operators compute.  Only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg may load it; the product path never does.  It
 * shares no code with the GPU library: its number formats, loops and
 * rounding are written here from the definitions.
 *
 * Sources (the operator documentation pages):
 *  [AG]  torch_npu.npu_all_gather_base_mm (Ascend PyTorch API page):
 *        "function" and "outputs" sections -- out = AllGather(input) @ x2 and
 *        the gathered input as the second output; "constraints" -- 2-D (m, k),
 *        (k, n), k in [256, 65535), x2 may be a transposed view.
 *  [A2A] aclnnAlltoAllQuantMatmul (CANN API page): "function" section, the
 *        dynamic-quant formula chain AlltoAll -> permute(1, 0, 2) -> Quant(
 *        permutedOut * x1Scale) -> int8 matmul -> x x1_scale x x2_scale -> + bias.
 *  [MC2] hyper_parallel tensor_parallel/mc2.py (coverage listing): module
 *        docstring and AllGatherMatmulFunction.backward -- dX = dY @ W
 *        (reduce-scattered across ranks), dW = dY^T @ AllGather(X);
 *        MatmulReduceScatterFunction.forward -- Y = ReduceScatter_m(X @ W^T).
 *  [QAR] QuantAllReduce README (ops-transformer mc2/quant_all_reduce):
 *        "function" formula output = Reduce(AllGather(scales) * AllGather(x))
 *        with sum, parameter table (scale shapes (bs, H/128) fp32 or
 *        (bs, H/64, 2) E8M0) and constraints (group size 128; mx).
 *
 * Precision: the float GEMMs are evaluated in fp64 (products exact, the sum
 * over k ascending) and rounded once to the output type (the definition, up
 * to summation order).  The dequantisation acc x s1 x s2 + bias is formed
 * exactly and rounded once.
 * The per-token quantisation takes its integer decisions in fp32, the
 * precision of the GPU kernel, because the pages fix none.  The int8 GEMM is
 * exact (int64, checked to fit int32).  QuantAllReduce sums fp64 products in
 * rank order; each product of an 8-bit code and its scale is exact in fp64.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off (no fast-math).  OpenMP splits
 * only independent output rows, so results do not depend on thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* dtype codes of this file (independent of any other header) */
enum { O_F32 = 0, O_F16 = 1, O_BF16 = 2, O_I8 = 3, O_I32 = 4, O_E4M3FN = 5, O_E5M2 = 6, O_E8M0 = 7 };

/* ------------------------------------------------------------------------ */
/* Number formats, from their published definitions.                         */
/* ------------------------------------------------------------------------ */

/* bf16: the upper 16 bits of an IEEE binary32. */
double orc_bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double orc_f16_to_f64(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 31)
    v = m ? NAN : INFINITY;
  else if (e == 0)
    v = ldexp((double)m, -24);
  else
    v = ldexp(1.0 + m / 1024.0, e - 15);
  return s ? -v : v;
}

/* OCP FLOAT8_E4M3FN: 1-4-3, bias 7, no infinities, S.1111.111 is NaN. */
double orc_e4m3fn_to_f64(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* OCP FLOAT8_E5M2: 1-5-2, bias 15, IEEE-style infinities and NaNs. */
double orc_e5m2_to_f64(uint8_t c) {
  int s = c >> 7, e = (c >> 2) & 31, m = c & 3;
  double v;
  if (e == 31)
    v = m ? NAN : INFINITY;
  else if (e == 0)
    v = ldexp((double)m, -16);
  else
    v = ldexp(1.0 + m / 4.0, e - 15);
  return s ? -v : v;
}

/* OCP FLOAT8_E8M0 (MX shared scale): 2^(b - 127); 0xFF is NaN. */
double orc_e8m0_to_f64(uint8_t b) { return b == 0xFF ? NAN : ldexp(1.0, (int)b - 127); }

/*
 * Round x to the binary format with p significand bits (implicit bit
 * included), minimum normal exponent emin and maximum exponent emax, ties to
 * even, overflow to infinity.  Returns the rounded value as a double.
 */
static double round_to_format(double x, int p, int emin, int emax) {
  if (isnan(x) || isinf(x) || x == 0.0) return x;
  double a = fabs(x);
  int e;
  frexp(a, &e); /* a in [2^(e-1), 2^e) */
  int E = e - 1;
  if (E < emin) E = emin;                  /* subnormal spacing */
  double q = ldexp(1.0, E - (p - 1));      /* spacing of the format at a */
  double n = nearbyint(a / q);             /* exact scaling; ties to even */
  double v = n * q;
  double maxf = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
  if (v > maxf) v = INFINITY;
  return x < 0 ? -v : v;
}

/* fp64 -> bf16, round to nearest even (bf16 = 8 significand bits, binary32 range). */
uint16_t orc_f64_to_bf16(double x) {
  if (isnan(x)) return (uint16_t)(signbit(x) ? 0xFFC0 : 0x7FC0);
  float f = (float)round_to_format(x, 8, -126, 127); /* exact in binary32 */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

/* fp64 -> IEEE binary16, round to nearest even, overflow to infinity. */
uint16_t orc_f64_to_f16(double x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  if (isnan(x)) return sign | 0x7E00;
  double v = fabs(round_to_format(x, 11, -14, 15));
  if (isinf(v)) return sign | 0x7C00;
  if (v == 0.0) return sign;
  if (v < ldexp(1.0, -14)) return sign | (uint16_t)(v * ldexp(1.0, 24)); /* subnormal */
  int e;
  double m = frexp(v, &e); /* v = m 2^e, m in [0.5, 1) */
  int E = e - 1;
  uint16_t frac = (uint16_t)((m * 2.0 - 1.0) * 1024.0);
  return sign | (uint16_t)((E + 15) << 10) | frac;
}

/* fp64 -> binary32, round to nearest even (the C conversion). */
float orc_f64_to_f32(double x) { return (float)x; }

static double dec16(int dtype, uint16_t v) {
  return dtype == O_BF16 ? orc_bf16_to_f64(v) : orc_f16_to_f64(v);
}
static uint16_t enc16(int dtype, double v) {
  return dtype == O_BF16 ? orc_f64_to_bf16(v) : orc_f64_to_f16(v);
}

/* ------------------------------------------------------------------------ */
/* [AG] AllGather on dim 0, rank order: gather_out rows [i m_l, (i+1) m_l)    */
/* hold shard i.                                                             */
/* ------------------------------------------------------------------------ */
void orc_allgather(const void* const* shards, int r, int64_t m_local, int64_t row_bytes,
                   void* gather_out) {
  for (int i = 0; i < r; i++)
    memcpy((char*)gather_out + (size_t)i * m_local * row_bytes, shards[i],
           (size_t)m_local * row_bytes);
}

/*
 * out (m, n) = round(A @ B) for 16-bit float A and B.
 *   a_trans = 0: A stored (m, k) row-major;  1: A stored (k, m) row-major.
 *   b_trans = 0: B stored (k, n) row-major;  1: B stored (n, k) row-major.
 * The products of two 16-bit floats are exact in fp64; the sum runs over p
 * ascending in fp64 and is rounded once to the output dtype.
 */
void orc_matmul(const uint16_t* a, int a_trans, const uint16_t* b, int b_trans, int64_t m,
                int64_t n, int64_t k, int dtype, uint16_t* out) {
  double* bd = (double*)malloc(sizeof(double) * (size_t)(k * n > 0 ? k * n : 1));
  for (int64_t p = 0; p < k; p++)
    for (int64_t j = 0; j < n; j++) bd[p * n + j] = dec16(dtype, b_trans ? b[j * k + p] : b[p * n + j]);
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t i = 0; i < m; i++) {
    double* acc = (double*)calloc((size_t)(n > 0 ? n : 1), sizeof(double));
    for (int64_t p = 0; p < k; p++) {
      double av = dec16(dtype, a_trans ? a[p * m + i] : a[i * k + p]);
      const double* brow = bd + p * n;
      for (int64_t j = 0; j < n; j++) acc[j] += av * brow[j];
    }
    for (int64_t j = 0; j < n; j++) out[i * n + j] = enc16(dtype, acc[j]);
    free(acc);
  }
  free(bd);
}

/*
 * [AG] out = AllGather_m(shards) @ x2 and gather_out = AllGather_m(shards).
 * Written as the two steps of the definition: gather, then multiply.
 * gather_out may be NULL (the op's gather_output = false).
 */
void orc_allgather_matmul(const uint16_t* const* shards, int r, int64_t m_local, int64_t k,
                          const uint16_t* x2, int64_t n, int x2_trans, int dtype, uint16_t* out,
                          uint16_t* gather_out) {
  uint16_t* g = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(r * m_local * k > 0 ? r * m_local * k : 1));
  orc_allgather((const void* const*)shards, r, m_local, k * (int64_t)sizeof(uint16_t), g);
  orc_matmul(g, 0, x2, x2_trans, r * m_local, n, k, dtype, out);
  if (gather_out) memcpy(gather_out, g, sizeof(uint16_t) * (size_t)(r * m_local * k));
  free(g);
}

/* ------------------------------------------------------------------------ */
/* [MC2] MatmulReduceScatter, the share of one rank.                         */
/* ------------------------------------------------------------------------ */

/*
 * Y = ReduceScatter_m(x @ x2) as rank `rank` of r sees it (the row-parallel
 * forward passes x2 = W^T; the backward dX = ReduceScatter_m(dY @ W)):
 *   partial = round(x @ x2), (m, n): this rank's matmul output, in the
 *             input dtype like any matmul output;
 *   out     = round(P_0 + P_1 + ... + P_{r-1}), (m / r, n), where P_j is
 *             block `rank` (rows [rank m/r, (rank+1) m/r)) of rank j's
 *             partial: recv[j] for j != rank (what rank j sent) and this
 *             rank's own partial for j == rank.  The sum runs in rank order
 *             in fp64 and is rounded once to the dtype.
 * recv[rank] is not read.  x2_trans: x2 stored (n, k) row-major.
 */
void orc_matmul_reduce_scatter(const uint16_t* x, const uint16_t* x2, int x2_trans, int r, int rank,
                               int64_t m, int64_t k, int64_t n, const uint16_t* const* recv, int dtype,
                               uint16_t* partial, uint16_t* out) {
  orc_matmul(x, 0, x2, x2_trans, m, n, k, dtype, partial);
  const int64_t rows = m / r;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < rows; t++)
    for (int64_t c = 0; c < n; c++) {
      double sum = 0.0;
      for (int j = 0; j < r; j++) {
        const uint16_t v = j == rank ? partial[(rank * rows + t) * n + c] : recv[j][t * n + c];
        sum += dec16(dtype, v);
      }
      out[t * n + c] = enc16(dtype, sum);
    }
}

/* ------------------------------------------------------------------------ */
/* [MC2] The tensor-parallel linear layer's bias and its gradient.           */
/* ------------------------------------------------------------------------ */

/*
 * AllGatherMatmulFunction.forward and MatmulReduceScatterFunction.forward add
 * the bias to the fused op's output (the fused op itself takes no non-zero
 * bias): y[i][j] = round(y[i][j] + bias[j]), the sum of two 16-bit values
 * formed in fp64 (exact) and rounded once, in place on y (m, n).
 */
void orc_add_bias(uint16_t* y, const uint16_t* bias, int64_t m, int64_t n, int dtype) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < m; i++)
    for (int64_t j = 0; j < n; j++) y[i * n + j] = enc16(dtype, dec16(dtype, y[i * n + j]) + dec16(dtype, bias[j]));
}

/*
 * grad_bias = grad_out.sum(dim=0) (both backward functions of the listing):
 * gb[j] = round(sum over i ascending of dy[i][j]), the sum in fp64 (exact as
 * long as a column's values span fewer than 53 - 8 - log2(m) binades) and
 * rounded once to the dtype.
 */
void orc_bias_grad(const uint16_t* dy, int64_t m, int64_t n, int dtype, uint16_t* gb) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; j++) {
    double s = 0.0;
    for (int64_t i = 0; i < m; i++) s += dec16(dtype, dy[i * n + j]);
    gb[j] = enc16(dtype, s);
  }
}

/* ------------------------------------------------------------------------ */
/* [A2A] AlltoAllQuantMatmul, dynamic per-token A16W8.                       */
/* ------------------------------------------------------------------------ */

/*
 * permutedOut = x1.view(r, bs/r, h).permute(1, 0, 2).view(bs/r, r h):
 *   P[t][j h + c] = x1[j (bs/r) + t][c].
 */
void orc_permute(const uint16_t* x1, int r, int64_t bs, int64_t h, uint16_t* p) {
  int64_t t_count = bs / r;
  for (int64_t t = 0; t < t_count; t++)
    for (int j = 0; j < r; j++)
      for (int64_t c = 0; c < h; c++) p[t * (r * h) + j * h + c] = x1[(j * t_count + t) * h + c];
}

/*
 * Quant(permutedOut * x1Scale), per token (row), symmetric int8:
 *   y      = P * smooth              (fp32; exact: two 8-bit significands)
 *   amax_t = max_c |y[t][c]|
 *   s1_t   = amax_t / 127            (fp32 division, round to nearest)
 *   q      = clamp(rint(y / s1_t), -127, 127)   (fp32 division, ties to even)
 * An all-zero row gives s1 = 0 and q = 0.  smooth may be NULL (no smoothing).
 */
void orc_smooth_quant(const uint16_t* p, int64_t rows, int64_t cols, const uint16_t* smooth,
                      int dtype, int8_t* q, float* s1) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < rows; t++) {
    float* y = (float*)malloc(sizeof(float) * (size_t)(cols > 0 ? cols : 1));
    float amax = 0.0f;
    for (int64_t c = 0; c < cols; c++) {
      float pv = (float)dec16(dtype, p[t * cols + c]);
      float sv = smooth ? (float)dec16(dtype, smooth[c]) : 1.0f;
      y[c] = pv * sv;
      float av = fabsf(y[c]);
      if (av > amax) amax = av;
    }
    float s = amax / 127.0f;
    s1[t] = s;
    for (int64_t c = 0; c < cols; c++) {
      int v = 0;
      if (amax > 0.0f) {
        float rq = rintf(y[c] / s);
        if (rq > 127.0f) rq = 127.0f;
        if (rq < -127.0f) rq = -127.0f;
        v = (int)rq;
      }
      q[t * cols + c] = (int8_t)v;
    }
    free(y);
  }
}

/*
 * acc (m, n) = q (m, k) @ x2 (k, n), both int8 row-major, exact.
 * Returns the number of entries whose exact value does not fit int32.
 */
int64_t orc_int8_matmul(const int8_t* q, const int8_t* x2, int64_t m, int64_t n, int64_t k,
                        int32_t* acc) {
  int64_t overflow = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : overflow)
  for (int64_t i = 0; i < m; i++) {
    int64_t* row = (int64_t*)calloc((size_t)(n > 0 ? n : 1), sizeof(int64_t));
    for (int64_t p = 0; p < k; p++) {
      int64_t qv = q[i * k + p];
      const int8_t* brow = x2 + p * n;
      for (int64_t j = 0; j < n; j++) row[j] += qv * (int64_t)brow[j];
    }
    for (int64_t j = 0; j < n; j++) {
      if (row[j] > INT32_MAX || row[j] < INT32_MIN) overflow++;
      acc[i * n + j] = (int32_t)row[j];
    }
    free(row);
  }
  return overflow;
}

/*
 * Exact rounding of a value given as an integer significand and a power of
 * two: (-1)^neg (N + t) 2^E with N > 0 and 0 <= t < 1, where t is known only
 * as zero (sticky = 0) or strictly between 0 and 1 (sticky = 1).  Rounds to
 * the binary format with p significand bits, smallest normal exponent emin
 * and largest exponent emax, ties to even, overflow to infinity, and returns
 * the result as a double (exact: at most 11 significant bits).
 */
static double round_exact(int neg, unsigned __int128 N, int E, int sticky, int p, int emin, int emax) {
  int nb = 0;
  for (unsigned __int128 t = N; t; t >>= 1) nb++;
  const int lead = nb - 1 + E;                           /* exponent of N's leading bit */
  const int ulp = (lead < emin ? emin : lead) - (p - 1); /* exponent of the format's last place */
  const int drop = ulp - E;                              /* low bits of N below that place */
  unsigned __int128 q;
  if (drop <= 0) {
    q = N << -drop; /* N fits in p bits at this scale; t < 1 ulp of N is below half a place */
  } else if (drop > nb) {
    q = 0; /* below half of the last place */
  } else {
    q = drop == 128 ? 0 : N >> drop;
    const unsigned __int128 rem = N - (q << drop), half = (unsigned __int128)1 << (drop - 1);
    if (rem > half || (rem == half && (sticky || (q & 1)))) q += 1;
  }
  double v = ldexp((double)q, ulp);
  if (v > ldexp(2.0 - ldexp(1.0, 1 - p), emax)) v = INFINITY;
  return neg ? -v : v;
}

/* x = M 2^E with M an odd integer (or 0) of at most 24 bits (any binary32 value). */
static void split_odd(double x, int64_t* M, int* E) {
  int e;
  double f = frexp(x, &e); /* x = f 2^e, |f| in [0.5, 1) */
  int64_t m = (int64_t)ldexp(f, 24);
  e -= 24;
  while (m != 0 && (m & 1) == 0) {
    m /= 2;
    e++;
  }
  *M = m;
  *E = e;
}

static int bitlen128(unsigned __int128 v) {
  int n = 0;
  for (; v; v >>= 1) n++;
  return n;
}

/*
 * output = output_quant x x1_scale x x2_scale + bias, per token x per channel,
 * rounded once from its exact value to out_dtype (bf16 or fp16): acc x s1 x s2
 * is an integer of at most 31 + 24 + 24 bits times a power of two, formed
 * exactly in 128-bit integers, and the bias (a 16-bit float) is added
 * exactly as well.  When the sum would not fit 128 bits, the two terms lie
 * so far apart that the smaller one is below the last of 16 zero bits
 * appended to the larger one: it then only decides the direction of
 * rounding and enters as a sticky bit.  bias may be NULL (zero).
 * Non-finite scales or bias fall back to fp64 arithmetic (NaN and infinity
 * propagate).
 */
static double dequant_exact(int32_t acc, float s1, float s2, double bias, int dtype) {
  const int p = dtype == O_BF16 ? 8 : 11, emin = dtype == O_BF16 ? -126 : -14, emax = dtype == O_BF16 ? 127 : 15;
  if (!isfinite(s1) || !isfinite(s2) || !isfinite(bias)) return (double)acc * s1 * s2 + bias;
  int64_t M1, M2, Mb;
  int E1, E2, Eb;
  split_odd(s1, &M1, &E1);
  split_odd(s2, &M2, &E2);
  split_odd(bias, &Mb, &Eb);
  const __int128 P = (__int128)acc * M1 * M2; /* |P| < 2^79 */
  const int EP = E1 + E2;
  if (P == 0 && Mb == 0) return (double)acc * s1 * s2 + bias; /* zeros: exact, IEEE signs */
  if (P == 0) return round_exact(Mb < 0, (unsigned __int128)(Mb < 0 ? -Mb : Mb), Eb, 0, p, emin, emax);
  if (Mb == 0) return round_exact(P < 0, (unsigned __int128)(P < 0 ? -P : P), EP, 0, p, emin, emax);
  /* both non-zero: hi is the term with the larger exponent, lo the other */
  __int128 hi = P, lo = Mb;
  int ehi = EP, elo = Eb;
  if (Eb > EP) {
    hi = Mb;
    lo = P;
    ehi = Eb;
    elo = EP;
  }
  const int d = ehi - elo;
  const int bh = bitlen128((unsigned __int128)(hi < 0 ? -hi : hi));
  if (bh + d <= 125) { /* hi 2^d + lo fits: exact */
    const __int128 S = hi * ((__int128)1 << d) + lo;
    if (S == 0) return 0.0;
    return round_exact(S < 0, (unsigned __int128)(S < 0 ? -S : S), elo, 0, p, emin, emax);
  }
  /* Here d > 125 - bh.  If hi is the product (bh <= 79), lo is the bias (at most 11
     bits) and d > 46; if hi is the bias (bh <= 11), lo is the product (at most 79
     bits) and d > 114.  Either way |lo| < 2^(d - 16): below one unit of |hi| 2^16 at
     exponent ehi - 16, so the value is |hi| 2^16 plus (same sign) or minus (opposite
     sign) a fraction of that unit. */
  const unsigned __int128 H = (unsigned __int128)(hi < 0 ? -hi : hi) << 16;
  const int same = (hi < 0) == (lo < 0);
  return round_exact(hi < 0, same ? H : H - 1, ehi - 16, 1, p, emin, emax);
}

void orc_dequant(const int32_t* acc, const float* s1, const float* s2, const uint16_t* bias,
                 int64_t m, int64_t n, int out_dtype, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < m; i++)
    for (int64_t j = 0; j < n; j++) {
      const double b = bias ? dec16(out_dtype, bias[j]) : 0.0;
      out[i * n + j] = enc16(out_dtype, dequant_exact(acc[i * n + j], s1[i], s2[j], b, out_dtype));
    }
}

/*
 * The whole chain for x1 of shape (bs, h) on r ranks.  Intermediate outputs
 * (permuted, q, s1, acc) are returned when the pointers are non-NULL.
 * Returns the int32 overflow count of the matmul.
 */
int64_t orc_alltoall_quant_matmul(const uint16_t* x1, int r, int64_t bs, int64_t h, int dtype,
                                  const int8_t* x2, int64_t n, const float* x2_scale,
                                  const uint16_t* smooth, const uint16_t* bias, uint16_t* out,
                                  uint16_t* permuted, int8_t* q_out, float* s1_out,
                                  int32_t* acc_out) {
  int64_t rows = bs / r, cols = (int64_t)r * h;
  uint16_t* p = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(rows * cols));
  int8_t* q = (int8_t*)malloc((size_t)(rows * cols));
  float* s1 = (float*)malloc(sizeof(float) * (size_t)rows);
  int32_t* acc = (int32_t*)malloc(sizeof(int32_t) * (size_t)(rows * n));
  orc_permute(x1, r, bs, h, p);
  orc_smooth_quant(p, rows, cols, smooth, dtype, q, s1);
  int64_t ovf = orc_int8_matmul(q, x2, rows, n, cols, acc);
  orc_dequant(acc, s1, x2_scale, bias, rows, n, dtype, out);
  if (permuted) memcpy(permuted, p, sizeof(uint16_t) * (size_t)(rows * cols));
  if (q_out) memcpy(q_out, q, (size_t)(rows * cols));
  if (s1_out) memcpy(s1_out, s1, sizeof(float) * (size_t)rows);
  if (acc_out) memcpy(acc_out, acc, sizeof(int32_t) * (size_t)(rows * n));
  free(p);
  free(q);
  free(s1);
  free(acc);
  return ovf;
}

/*
 * Full-quantisation variant (aclnnAlltoAllQuantMatmul page, "function"
 * formulas, full-quant case): x1 arrives already int8 with one scale per
 * token of the permuted matrix, so
 *   P   = AlltoAll + permute of x1 (int8 bytes, the same addressing as above)
 *   acc = P @ x2                         (exact, int32)
 *   out = acc * x1_scale * x2_scale + bias
 * The page prints the matmul as "x1 @ x2"; since the permute is defined just
 * before it and the shapes only match after it, the product is read as
 * P @ x2.  Returns the int32 overflow count.
 */
void orc_permute_i8(const int8_t* x1, int r, int64_t bs, int64_t h, int8_t* p) {
  int64_t t_count = bs / r;
  for (int64_t t = 0; t < t_count; t++)
    for (int j = 0; j < r; j++)
      for (int64_t c = 0; c < h; c++) p[t * (r * h) + j * h + c] = x1[(j * t_count + t) * h + c];
}

int64_t orc_alltoall_quant_matmul_static(const int8_t* x1, int r, int64_t bs, int64_t h, const float* x1_scale,
                                         const int8_t* x2, int64_t n, const float* x2_scale, const uint16_t* bias,
                                         int dtype, uint16_t* out, int8_t* permuted, int32_t* acc_out) {
  int64_t rows = bs / r, cols = (int64_t)r * h;
  int8_t* p = (int8_t*)malloc((size_t)(rows * cols));
  int32_t* acc = (int32_t*)malloc(sizeof(int32_t) * (size_t)(rows * n));
  orc_permute_i8(x1, r, bs, h, p);
  int64_t ovf = orc_int8_matmul(p, x2, rows, n, cols, acc);
  orc_dequant(acc, x1_scale, x2_scale, bias, rows, n, dtype, out);
  if (permuted) memcpy(permuted, p, (size_t)(rows * cols));
  if (acc_out) memcpy(acc_out, acc, sizeof(int32_t) * (size_t)(rows * n));
  free(p);
  free(acc);
  return ovf;
}

/* ------------------------------------------------------------------------ */
/* [QAR] QuantAllReduce: output = sum over ranks of scale * x.               */
/* ------------------------------------------------------------------------ */

static double dec_x(int x_dtype, const void* x, int64_t e) {
  switch (x_dtype) {
    case O_I8: return (double)((const int8_t*)x)[e];
    case O_E4M3FN: return orc_e4m3fn_to_f64(((const uint8_t*)x)[e]);
    case O_E5M2: return orc_e5m2_to_f64(((const uint8_t*)x)[e]);
    default: return NAN;
  }
}

/*
 * x[i]: rank i's (rows, h) tensor; scales[i]: its scales.
 *   scale_dtype F32 (per-token per-group, group 128): scale index row*(h/128) + c/128.
 *   scale_dtype E8M0 (mx, block 32): the (rows, h/64, 2) tensor is the
 *     row-major packing of (rows, h/32), scale index row*(h/32) + c/32.
 * out[e] = sum_{i=0..r-1} dec(x_i[e]) * dec(scale_i[g(e)]), fp64 in rank
 * order, rounded once to out_dtype (F32, BF16 or F16).  Returns 0, or -1 on
 * an unsupported dtype combination.
 */
int orc_quant_all_reduce(const void* const* x, const void* const* scales, int r, int64_t rows,
                         int64_t h, int x_dtype, int scale_dtype, void* out, int out_dtype) {
  if (scale_dtype == O_F32 && !(x_dtype == O_I8 || x_dtype == O_E4M3FN || x_dtype == O_E5M2)) return -1;
  if (scale_dtype == O_E8M0 && !(x_dtype == O_E4M3FN || x_dtype == O_E5M2)) return -1;
  if (scale_dtype != O_F32 && scale_dtype != O_E8M0) return -1;
  if (out_dtype != O_F32 && out_dtype != O_BF16 && out_dtype != O_F16) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < rows; t++)
    for (int64_t c = 0; c < h; c++) {
      int64_t e = t * h + c;
      double sum = 0.0;
      for (int i = 0; i < r; i++) {
        double s = scale_dtype == O_F32 ? (double)((const float*)scales[i])[t * (h / 128) + c / 128]
                                        : orc_e8m0_to_f64(((const uint8_t*)scales[i])[t * (h / 32) + c / 32]);
        sum += dec_x(x_dtype, x[i], e) * s;
      }
      if (out_dtype == O_F32)
        ((float*)out)[e] = orc_f64_to_f32(sum);
      else
        ((uint16_t*)out)[e] = enc16(out_dtype, sum);
    }
  return 0;
}

/*
 * QuantReduceScatter, the share of rank `rank` of r (named beside
 * QuantAllReduce in its README's constraints; read as the reduce-scatter
 * form): rows [rank rows/r, (rank+1) rows/r) of the QuantAllReduce output,
 * with the same per-element sum.  out is (rows / r, h).
 */
int orc_quant_reduce_scatter(const void* const* x, const void* const* scales, int r, int rank, int64_t rows,
                             int64_t h, int x_dtype, int scale_dtype, void* out, int out_dtype) {
  const int64_t block = rows / r, row0 = (int64_t)rank * block;
  const int64_t scale_row_bytes = scale_dtype == O_F32 ? (h / 128) * 4 : h / 32;
  const void* xb[8];
  const void* sb[8];
  if (r < 1 || r > 8 || rows % r != 0) return -1;
  for (int i = 0; i < r; i++) {
    xb[i] = (const uint8_t*)x[i] + row0 * h;
    sb[i] = (const uint8_t*)scales[i] + row0 * scale_row_bytes;
  }
  return orc_quant_all_reduce(xb, sb, r, block, h, x_dtype, scale_dtype, out, out_dtype);
}

/* ------------------------------------------------------------------------ */
/* [A2A] int4 operands of A16W4 / A4W4.                                      */
/* ------------------------------------------------------------------------ */

/*
 * The constraints of the AlltoAllQuantMatmul page require N even for A16W4
 * and H and N even for A4W4, which fits two 4-bit codes per byte along the
 * last dimension.  Reading taken: two's-complement int4 codes (-8..7), value
 * 2i of a row in the low nibble of byte i and value 2i + 1 in the high
 * nibble.  n_values (even) codes from n_values / 2 bytes.
 */
void orc_unpack_int4(const uint8_t* packed, int64_t n_values, int8_t* out) {
  for (int64_t i = 0; i < n_values / 2; i++) {
    const int lo = packed[i] & 0xF, hi = packed[i] >> 4;
    out[2 * i] = (int8_t)(lo >= 8 ? lo - 16 : lo);
    out[2 * i + 1] = (int8_t)(hi >= 8 ? hi - 16 : hi);
  }
}

/* ------------------------------------------------------------------------ */
/* Array forms of the format routines (for the format tests).               */
/* ------------------------------------------------------------------------ */
int orc_decode_array(int dtype, int64_t n, const void* in, double* out) {
  for (int64_t i = 0; i < n; i++) {
    switch (dtype) {
      case O_F32: out[i] = (double)((const float*)in)[i]; break;
      case O_F16: out[i] = orc_f16_to_f64(((const uint16_t*)in)[i]); break;
      case O_BF16: out[i] = orc_bf16_to_f64(((const uint16_t*)in)[i]); break;
      case O_I8: out[i] = (double)((const int8_t*)in)[i]; break;
      case O_E4M3FN: out[i] = orc_e4m3fn_to_f64(((const uint8_t*)in)[i]); break;
      case O_E5M2: out[i] = orc_e5m2_to_f64(((const uint8_t*)in)[i]); break;
      case O_E8M0: out[i] = orc_e8m0_to_f64(((const uint8_t*)in)[i]); break;
      default: return -1;
    }
  }
  return 0;
}

int orc_encode_array(int dtype, int64_t n, const double* in, void* out) {
  for (int64_t i = 0; i < n; i++) {
    switch (dtype) {
      case O_F32: ((float*)out)[i] = orc_f64_to_f32(in[i]); break;
      case O_F16: ((uint16_t*)out)[i] = orc_f64_to_f16(in[i]); break;
      case O_BF16: ((uint16_t*)out)[i] = orc_f64_to_bf16(in[i]); break;
      default: return -1;
    }
  }
  return 0;
}

/* Threads the OpenMP loops above use (for reporting the CPU baseline). */
#ifdef _OPENMP
#include <omp.h>
int orc_num_threads(void) { return omp_get_max_threads(); }
#else
int orc_num_threads(void) { return 1; }
#endif
