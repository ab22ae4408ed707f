/*
 * Sanitizer driver for the oracle (test infrastructure): calls every entry
 * point of oracle/mc2_oracle.c on small inputs in exactly-sized heap
 * buffers, so that an AddressSanitizer / UndefinedBehaviorSanitizer build
 * reports any out-of-bounds access, overflow or invalid shift.  The values
 * are not checked here (the pin tests do that); exit status 0 means clean.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

enum { F32 = 0, F16 = 1, BF16 = 2, I8 = 3, E4M3FN = 5, E5M2 = 6, E8M0 = 7 };

void orc_allgather(const void* const* shards, int r, int64_t m_local, int64_t row_bytes, void* gather_out);
void orc_matmul(const uint16_t* a, int a_trans, const uint16_t* b, int b_trans, int64_t m, int64_t n, int64_t k,
                int dtype, uint16_t* out);
void orc_allgather_matmul(const uint16_t* const* shards, int r, int64_t m_local, int64_t k, const uint16_t* x2,
                          int64_t n, int x2_trans, int dtype, uint16_t* out, uint16_t* gather_out);
void orc_matmul_reduce_scatter(const uint16_t* x, const uint16_t* x2, int x2_trans, int r, int rank, int64_t m,
                               int64_t k, int64_t n, const uint16_t* const* recv, int dtype, uint16_t* partial,
                               uint16_t* out);
void orc_add_bias(uint16_t* y, const uint16_t* bias, int64_t m, int64_t n, int dtype);
void orc_bias_grad(const uint16_t* dy, int64_t m, int64_t n, int dtype, uint16_t* gb);
void orc_permute(const uint16_t* x1, int r, int64_t bs, int64_t h, uint16_t* p);
void orc_smooth_quant(const uint16_t* p, int64_t rows, int64_t cols, const uint16_t* smooth, int dtype, int8_t* q,
                      float* s1);
int64_t orc_int8_matmul(const int8_t* q, const int8_t* x2, int64_t m, int64_t n, int64_t k, int32_t* acc);
void orc_dequant(const int32_t* acc, const float* s1, const float* s2, const uint16_t* bias, int64_t m, int64_t n,
                 int out_dtype, uint16_t* out);
int64_t orc_alltoall_quant_matmul(const uint16_t* x1, int r, int64_t bs, int64_t h, int dtype, const int8_t* x2,
                                  int64_t n, const float* x2_scale, const uint16_t* smooth, const uint16_t* bias,
                                  uint16_t* out, uint16_t* permuted, int8_t* q_out, float* s1_out, int32_t* acc_out);
void orc_permute_i8(const int8_t* x1, int r, int64_t bs, int64_t h, int8_t* p);
int64_t orc_alltoall_quant_matmul_static(const int8_t* x1, int r, int64_t bs, int64_t h, const float* x1_scale,
                                         const int8_t* x2, int64_t n, const float* x2_scale, const uint16_t* bias,
                                         int dtype, uint16_t* out, int8_t* permuted, int32_t* acc_out);
int orc_quant_all_reduce(const void* const* x, const void* const* scales, int r, int64_t rows, int64_t h,
                         int x_dtype, int scale_dtype, void* out, int out_dtype);
int orc_quant_reduce_scatter(const void* const* x, const void* const* scales, int r, int rank, int64_t rows,
                             int64_t h, int x_dtype, int scale_dtype, void* out, int out_dtype);
int orc_decode_array(int dtype, int64_t n, const void* in, double* out);
int orc_encode_array(int dtype, int64_t n, const double* in, void* out);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return (uint32_t)(state >> 16);
}
/* random finite 16-bit floats of moderate size, int8 codes, fp8 codes */
static uint16_t* h16(size_t n, int dtype) {
  uint16_t* p = malloc(n * 2);
  for (size_t i = 0; i < n; i++) {
    uint16_t sign = (uint16_t)((rnd() & 1) << 15);
    p[i] = dtype == BF16 ? (uint16_t)(sign | (0x3C00 + rnd() % 0x0700)) : (uint16_t)(sign | (0x3000 + rnd() % 0x1400));
  }
  return p;
}
static int8_t* i8(size_t n) {
  int8_t* p = malloc(n);
  for (size_t i = 0; i < n; i++) p[i] = (int8_t)((int)(rnd() % 255) - 127);
  return p;
}
static uint8_t* u8(size_t n, unsigned lo, unsigned span) {
  uint8_t* p = malloc(n);
  for (size_t i = 0; i < n; i++) p[i] = (uint8_t)(lo + rnd() % span);
  return p;
}
static float* f32(size_t n, float a, float b) {
  float* p = malloc(n * 4);
  for (size_t i = 0; i < n; i++) p[i] = a + (b - a) * (float)(rnd() % 1000000) / 1e6f;
  return p;
}

int main(void) {
  for (int dt = F16; dt <= BF16; dt++) {
    /* AllGatherMatmul, matmul in every layout, reduce-scatter, bias */
    const int r = 4;
    const int64_t ml = 3, k = 300, n = 7, m = r * ml;
    uint16_t* sh[4];
    for (int i = 0; i < r; i++) sh[i] = h16((size_t)(ml * k), dt);
    uint16_t* x2 = h16((size_t)(k * n), dt);
    uint16_t* out = malloc((size_t)(m * n) * 2);
    uint16_t* g = malloc((size_t)(m * k) * 2);
    orc_allgather_matmul((const uint16_t* const*)sh, r, ml, k, x2, n, 0, dt, out, g);
    orc_allgather_matmul((const uint16_t* const*)sh, r, ml, k, x2, n, 1, dt, out, NULL);
    orc_allgather((const void* const*)sh, r, ml, k * 2, g);
    for (int at = 0; at < 2; at++)
      for (int bt = 0; bt < 2; bt++) orc_matmul(g, at, x2, bt, m, n, k, dt, out); /* same sizes, other layouts */
    uint16_t* part = malloc((size_t)(m * n) * 2);
    uint16_t* rs = malloc((size_t)(ml * n) * 2);
    uint16_t* recv[4];
    for (int j = 0; j < r; j++) recv[j] = h16((size_t)(ml * n), dt);
    orc_matmul_reduce_scatter(g, x2, 0, r, 2, m, k, n, (const uint16_t* const*)recv, dt, part, rs);
    uint16_t* bias = h16((size_t)n, dt);
    orc_add_bias(out, bias, m, n, dt);
    orc_bias_grad(out, m, n, dt, bias);
    for (int i = 0; i < r; i++) free(sh[i]);
    for (int j = 0; j < r; j++) free(recv[j]);
    free(x2), free(out), free(g), free(part), free(rs), free(bias);

    /* AlltoAllQuantMatmul: dynamic and static, steps and chain */
    const int64_t bs = 8, h = 24, nn = 5, rows = bs / r, cols = r * h;
    uint16_t* x1 = h16((size_t)(bs * h), dt);
    uint16_t* sm = h16((size_t)cols, dt);
    uint16_t* p = malloc((size_t)(rows * cols) * 2);
    int8_t* q = malloc((size_t)(rows * cols));
    float* s1 = malloc((size_t)rows * 4);
    int8_t* w8 = i8((size_t)(cols * nn));
    int32_t* acc = malloc((size_t)(rows * nn) * 4);
    float* s2 = f32((size_t)nn, 1e-3f, 1e-2f);
    uint16_t* b2 = h16((size_t)nn, dt);
    uint16_t* o2 = malloc((size_t)(rows * nn) * 2);
    orc_permute(x1, r, bs, h, p);
    orc_smooth_quant(p, rows, cols, sm, dt, q, s1);
    orc_smooth_quant(p, rows, cols, NULL, dt, q, s1);
    orc_int8_matmul(q, w8, rows, nn, cols, acc);
    orc_dequant(acc, s1, s2, b2, rows, nn, dt, o2);
    orc_dequant(acc, s1, s2, NULL, rows, nn, dt, o2);
    orc_alltoall_quant_matmul(x1, r, bs, h, dt, w8, nn, s2, sm, b2, o2, p, q, s1, acc);
    orc_alltoall_quant_matmul(x1, r, bs, h, dt, w8, nn, s2, NULL, NULL, o2, NULL, NULL, NULL, NULL);
    int8_t* x8 = i8((size_t)(bs * h));
    orc_permute_i8(x8, r, bs, h, q);
    orc_alltoall_quant_matmul_static(x8, r, bs, h, s1, w8, nn, s2, b2, dt, o2, q, acc);
    orc_alltoall_quant_matmul_static(x8, r, bs, h, s1, w8, nn, s2, NULL, dt, o2, NULL, NULL);
    /* dequant extremes: the exact 128-bit path with the widest products and far-apart terms */
    int32_t ea[4] = {INT32_MAX, INT32_MIN, 1, 0};
    float es1[1] = {16777215.0f}, es2[4] = {16777215.0f, 1e-38f, 3.4e38f, 0.5f};
    uint16_t eb[4] = {0x7BFF, 0x0001, 0x8001, 0x3C00}, eo[4];
    orc_dequant(ea, es1, es2, eb, 1, 4, dt, eo);
    free(x1), free(sm), free(p), free(q), free(s1), free(w8), free(acc), free(s2), free(b2), free(o2), free(x8);
  }
  /* QuantAllReduce / QuantReduceScatter: int8 + fp32 groups, fp8 + fp32 groups, fp8 + E8M0 */
  {
    const int r = 4;
    const int64_t rows = 8, h = 256, e = rows * h;
    const int outs[3] = {F32, BF16, F16};
    void *x[4], *sc[4];
    for (int kind = 0; kind < 3; kind++) {
      int xd = kind == 0 ? I8 : (kind == 1 ? E4M3FN : E5M2), sd = kind == 2 ? E8M0 : F32;
      for (int i = 0; i < r; i++) {
        x[i] = kind == 0 ? (void*)i8((size_t)e) : (void*)u8((size_t)e, 0, 120);
        sc[i] = sd == F32 ? (void*)f32((size_t)(e / 128), 1e-3f, 1e-2f) : (void*)u8((size_t)(e / 32), 119, 9);
      }
      for (int o = 0; o < 3; o++) {
        void* out = malloc((size_t)e * 4);
        void* blk = malloc((size_t)(e / r) * 4);
        if (orc_quant_all_reduce((const void* const*)x, (const void* const*)sc, r, rows, h, xd, sd, out, outs[o]))
          return 10;
        if (orc_quant_reduce_scatter((const void* const*)x, (const void* const*)sc, r, 3, rows, h, xd, sd, blk,
                                     outs[o]))
          return 11;
        free(out), free(blk);
      }
      for (int i = 0; i < r; i++) free(x[i]), free(sc[i]);
    }
  }
  /* every code of every format, both directions */
  {
    uint16_t codes[65536];
    double v[65536];
    for (int i = 0; i < 65536; i++) codes[i] = (uint16_t)i;
    for (int dt = F16; dt <= BF16; dt++) {
      if (orc_decode_array(dt, 65536, codes, v)) return 20;
      uint16_t back[65536];
      if (orc_encode_array(dt, 65536, v, back)) return 21;
    }
    uint8_t c8[256];
    for (int i = 0; i < 256; i++) c8[i] = (uint8_t)i;
    const int f8[4] = {I8, E4M3FN, E5M2, E8M0};
    for (int i = 0; i < 4; i++)
      if (orc_decode_array(f8[i], 256, c8, v)) return 22;
    float f[256];
    if (orc_encode_array(F32, 256, v, f) || orc_decode_array(F32, 256, f, v)) return 23;
  }
  puts("oracle driver: clean");
  return 0;
}
