// K1 with 256 x 256 tiles: the launches of the 16-bit GEMM (gemm16.hpp) for
// outputs of 256 such tiles or more (e.g. the row-parallel forward's
// 4096 x 4096 partial) with a K-contiguous B or an M-contiguous A.
// Each wavefront holds a 128 x 128 block of C, so its 256 fp32 accumulator
// registers live in AGPRs; the two-stage LDS ring (gemm_mfma.hpp,
// mainloop_fast with NS = 2) keeps the tile's staging within the LDS.
// Built as its own translation unit with the MFMAs in their AGPR form and a
// raised unroll limit, so each half step's 64 MFMAs unroll fully.
#include "gemm16.hpp"

namespace mc2 {

template <bool AK, bool BKM, int DT>
hipError_t launch_gemm16_256(const gemm::Problem& p, void* c, hipStream_t s) {
  return launch_cfg<256, 256, AK, BKM, DT>(p, c, s);
}

template hipError_t launch_gemm16_256<true, true, DT_BF16>(const gemm::Problem&, void*, hipStream_t);
template hipError_t launch_gemm16_256<false, true, DT_BF16>(const gemm::Problem&, void*, hipStream_t);
template hipError_t launch_gemm16_256<false, false, DT_BF16>(const gemm::Problem&, void*, hipStream_t);
template hipError_t launch_gemm16_256<true, true, DT_F16>(const gemm::Problem&, void*, hipStream_t);
template hipError_t launch_gemm16_256<false, true, DT_F16>(const gemm::Problem&, void*, hipStream_t);
template hipError_t launch_gemm16_256<false, false, DT_F16>(const gemm::Problem&, void*, hipStream_t);

}  // namespace mc2
