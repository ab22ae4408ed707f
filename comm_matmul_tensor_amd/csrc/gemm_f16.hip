// K1: the fp16 instantiations of the 16-bit float GEMM (gemm16.hpp); the
// entry points and the bf16 ones are in gemm_bf16.hip.
#include "gemm16.hpp"

namespace mc2 {

hipError_t launch_gemm16_f16(const GemmArgs& g, hipStream_t s) { return launch_gemm16_dt<DT_F16>(g, s); }

}  // namespace mc2
