// Sanitizer driver for libmc2's host-side argument validation (test
// infrastructure): runs every check of csrc/validate.cpp on valid and
// invalid arguments, so that an AddressSanitizer / UndefinedBehaviorSanitizer
// build reports any bad access or overflow (huge sizes included), and
// checks each returned status.  Fake pointers are never dereferenced.
#include <cstdint>
#include <cstdio>

#include "validate.hpp"

using namespace mc2;

static int failures = 0;
static void expect(mc2_status got, mc2_status want, const char* what) {
  if (got != want) {
    std::printf("%s: got %d, want %d (%s)\n", what, (int)got, (int)want, last_error_text());
    failures++;
  }
}

int main() {
  void* A = reinterpret_cast<void*>(0x10000);
  void* U = reinterpret_cast<void*>(0x10008);  // not 16-byte aligned
  const void* sh[8] = {A, A, A, A, A, A, A, A};
  const void* shn[8] = {A, nullptr, A, A, A, A, A, A};
  const void* own0[8] = {nullptr, A, A, A, A, A, A, A};  // received blocks of rank 0 (its own slot unused)
  const int64_t big = (int64_t)1 << 62;
  // AllGatherMatmul
  expect(check_allgather_matmul(sh, 8, 512, 4096, A, 1792, MC2_BF16, A, A, MC2_AG_FUSED_WRITE, 0), MC2_OK, "ag ok");
  expect(check_allgather_matmul(sh, 8, 512, 4096, A, 1792, MC2_BF16, A, A, MC2_AG_ARRIVAL, 7), MC2_OK, "ag arrival");
  expect(check_allgather_matmul(sh, 3, 512, 4096, A, 1792, MC2_BF16, A, A, 0, 0), MC2_ERR_SHAPE, "ag r=3");
  expect(check_allgather_matmul(shn, 8, 512, 4096, A, 1792, MC2_BF16, A, A, 0, 0), MC2_ERR_NULL, "ag null shard");
  expect(check_allgather_matmul(sh, 8, 512, 255, A, 1792, MC2_BF16, A, A, 0, 0), MC2_ERR_SHAPE, "ag k=255");
  expect(check_allgather_matmul(sh, 8, 512, 65535, A, 1792, MC2_BF16, A, A, 0, 0), MC2_ERR_SHAPE, "ag k=65535");
  expect(check_allgather_matmul(sh, 8, big, 4096, A, big, MC2_BF16, A, A, 0, 0), MC2_ERR_SHAPE, "ag huge");
  expect(check_allgather_matmul(sh, 8, 512, 4096, A, 1792, MC2_F32, A, A, 0, 0), MC2_ERR_DTYPE, "ag f32");
  expect(check_allgather_matmul(sh, 8, 512, 4096, A, 1792, MC2_BF16, A, nullptr, MC2_AG_ARRIVAL, 0), MC2_ERR_NULL,
         "ag arrival no gather");
  expect(check_allgather_matmul(sh, 8, 512, 4096, A, 1792, MC2_BF16, A, A, MC2_AG_ARRIVAL, 8), MC2_ERR_SHAPE,
         "ag arrival rank");
  expect(check_allgather_matmul(sh, 8, 512, 4096, U, 1792, MC2_BF16, A, A, 0, 0), MC2_ERR_ALIGN, "ag align");
  // backward pair
  expect(check_grad_input(A, A, 8192, 1792, 4096, MC2_BF16, A), MC2_OK, "dx ok");
  expect(check_grad_input(A, A, 8192, 100, 4096, MC2_BF16, A), MC2_ERR_SHAPE, "dx n_local");
  expect(check_grad_input(A, A, big, 1792, big, MC2_BF16, A), MC2_ERR_SHAPE, "dx huge");
  expect(check_grad_weight(A, A, 8192, 1792, 4096, MC2_F16, A), MC2_OK, "dw ok");
  expect(check_grad_weight(A, nullptr, 8192, 1792, 4096, MC2_F16, A), MC2_ERR_NULL, "dw null");
  expect(check_grad_weight(A, A, 0, 1792, 4096, MC2_F16, A), MC2_ERR_SHAPE, "dw empty");
  // MatmulReduceScatter
  expect(check_matmul_reduce_scatter(A, A, 8, 0, 4096, 1792, 4096, MC2_BF16, own0, A, A), MC2_OK, "rs ok (own null)");
  expect(check_matmul_reduce_scatter(A, A, 8, 1, 4096, 1792, 4096, MC2_BF16, shn, A, A), MC2_OK, "rs ok");
  expect(check_matmul_reduce_scatter(A, A, 8, 2, 4096, 1792, 4096, MC2_BF16, shn, A, A), MC2_ERR_NULL, "rs null");
  expect(check_matmul_reduce_scatter(A, A, 8, 0, 4095, 1792, 4096, MC2_BF16, own0, A, A), MC2_ERR_SHAPE, "rs m%r");
  expect(check_matmul_reduce_scatter(A, A, 8, 9, 4096, 1792, 4096, MC2_BF16, sh, A, A), MC2_ERR_SHAPE, "rs rank");
  // bias and its gradient
  expect(check_bias("x", A), MC2_OK, "bias ok");
  expect(check_bias("x", nullptr), MC2_ERR_NULL, "bias null");
  expect(check_bias("x", U), MC2_ERR_ALIGN, "bias align");
  expect(check_bias_grad(A, 8192, 1792, MC2_BF16, A), MC2_OK, "gb ok");
  expect(check_bias_grad(A, big, 1792, MC2_BF16, A), MC2_ERR_SHAPE, "gb huge");
  expect(check_bias_grad(A, 8192, 1792, MC2_I8, A), MC2_ERR_DTYPE, "gb dtype");
  // AlltoAllQuantMatmul
  expect(check_alltoall_sizes(8, 8192, 4096, 7168), MC2_OK, "a2a sizes ok");
  expect(check_alltoall_sizes(8, 8192, 4376, 7168), MC2_ERR_SHAPE, "a2a r*h > 35000");
  expect(check_alltoall_sizes(8, 8191, 4096, 7168), MC2_ERR_SHAPE, "a2a bs%r");
  expect(check_alltoall_sizes(8, big, 4096, big), MC2_ERR_SHAPE, "a2a huge");
  expect(check_alltoall_sizes(8, 8192, big, 7168), MC2_ERR_SHAPE, "a2a huge h");
  expect(check_alltoall_quant_matmul(A, 8, 8192, 4096, MC2_BF16, A, 7168, A, A, A, A, nullptr, nullptr, nullptr,
                                     nullptr, A, 100, 100),
         MC2_OK, "a2a ok");
  expect(check_alltoall_quant_matmul(A, 8, 8192, 4096, MC2_BF16, A, 7168, A, A, A, A, nullptr, nullptr, nullptr,
                                     nullptr, A, 99, 100),
         MC2_ERR_WORKSPACE, "a2a workspace");
  expect(check_alltoall_quant_matmul_static(A, 8, 8192, 4096, A, A, 7168, A, A, A, MC2_BF16, nullptr, nullptr), MC2_OK,
         "a8w8 ok");
  expect(check_alltoall_quant_matmul_static(A, 8, 8192, 4096, nullptr, A, 7168, A, A, A, MC2_BF16, nullptr, nullptr),
         MC2_ERR_NULL, "a8w8 no scale");
  // QuantAllReduce / QuantReduceScatter
  expect(check_quant_all_reduce(sh, sh, 8, 8192, 7168, MC2_I8, MC2_F32, A, MC2_F32), MC2_OK, "qar ok");
  expect(check_quant_all_reduce(sh, sh, 8, 8192, 7168, MC2_F8E4M3FN, MC2_E8M0, A, MC2_BF16), MC2_OK, "qar mx");
  expect(check_quant_all_reduce(sh, sh, 8, 8192, 7000, MC2_I8, MC2_F32, A, MC2_F32), MC2_ERR_SHAPE, "qar h%128");
  expect(check_quant_all_reduce(sh, sh, 8, big, 7168, MC2_I8, MC2_F32, A, MC2_F32), MC2_ERR_SHAPE, "qar huge");
  expect(check_quant_reduce_scatter(sh, sh, 8, 3, 8192, 7168, MC2_I8, MC2_F32, A, MC2_F32), MC2_OK, "qrs ok");
  expect(check_quant_reduce_scatter(sh, sh, 8, 8, 8192, 7168, MC2_I8, MC2_F32, A, MC2_F32), MC2_ERR_SHAPE, "qrs rank");
  if (failures) return 1;
  std::puts("validate driver: clean");
  return 0;
}
