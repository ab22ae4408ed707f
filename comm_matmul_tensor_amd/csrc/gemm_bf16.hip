// K1 entry points and the bf16 instantiations; the fp16 ones are compiled in
// gemm_f16.hip (same implementation, gemm16.hpp) so the two build in parallel.
#include "gemm16.hpp"

namespace mc2 {

// Arrival mode needs AK (A K-major); B may be either layout.
int gemm16_tile_rows(int64_t m, int64_t n, int b_kmajor) {
  const TileChoice* t = b_kmajor ? tiles16<true, true>() : tiles16<true, false>();
  return t[pick_tile(m, n, t, kNumTiles3)].bm;
}

hipError_t launch_gemm16(const GemmArgs& g, hipStream_t s) {
  if (g.m < 1 || g.n < 1 || g.k < 1 || g.num_parts < 1 || g.num_parts > kMaxRanks) return hipErrorInvalidValue;
  if (g.num_parts * g.rows_per_part != g.m) return hipErrorInvalidValue;
  if (g.gather_out && !g.a_kmajor) return hipErrorInvalidValue;
  if (g.ready_flags) {
    const int bm = gemm16_tile_rows(g.m, g.n, g.b_kmajor);
    if (!g.gather_out || !g.status_flag || !g.a_kmajor || g.rows_chunk < bm || g.rows_chunk % bm != 0 ||
        g.slabs < 1 || g.slab_cols < 1 || g.slab_cols % 64 != 0 || (int64_t)g.slabs * g.slab_cols < g.k ||
        g.first_row_tile < 0 || (int64_t)g.first_row_tile * bm >= g.m)
      return hipErrorInvalidValue;
  }
  if (g.rs_out) {
    if (g.ready_flags || g.gather_out || g.rs_ranks < 1 || g.rs_ranks > kMaxRanks || g.rs_rank < 0 ||
        g.rs_rank >= g.rs_ranks || g.rs_row0 < 0 || g.rs_rows < 1 || g.rs_row0 + g.rs_rows > g.m)
      return hipErrorInvalidValue;
    for (int j = 0; j < g.rs_ranks; j++)
      if (j != g.rs_rank && !g.rs_recv[j]) return hipErrorInvalidValue;
  }
  if (g.dtype != DT_BF16 && g.dtype != DT_F16) return hipErrorInvalidValue;
  return g.dtype == DT_BF16 ? launch_gemm16_dt<DT_BF16>(g, s) : launch_gemm16_f16(g, s);
}

}  // namespace mc2
