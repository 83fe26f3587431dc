// Launcher of the matrix-core (prefill) path: 64-row tiles here, 128-row
// tiles in gemm_prefill_128.hip (its own translation unit, compiled with the
// max-ILP instruction scheduler; see build.py).  The kernels are in
// gemm_prefill_tiles.hpp.
#include "gemm_prefill_tiles.hpp"

namespace milo {

int32_t launch_gemm_prefill(const milo_gemm_desc* d, const GemmPlan& p, char* ws, hipStream_t st) {
  if (!p.pre_launch) return MILO_OK;
  GemmArgs a = make_gemm_args(d, p, ws);
  // 128-row tiles where experts average 256 rows or more, else 64-row tiles
  // (less padding and twice the blocks for mid-sized experts)
  const dim3 grid(d->n_w == 2 ? (p.n_tiles + 1) / 2 : (p.n_tiles + 3) / 4, p.pre_tiles);
  if (p.pre_bm == 128) return launch_gemm_prefill_128(a, d->n_w, grid, st);
  const size_t lds = prefill_lds(64);
  const int n_groups = grid.x;
  const int items_bound = n_groups * p.pre_tiles;
  const int pgrid = items_bound < p.pre_slots ? items_bound : p.pre_slots;
  if (d->n_w == 2 && a.x_bytes_32) {
    if (a.lrq) hipLaunchKernelGGL((gemm_prefill_persistent<2, true>), dim3(pgrid), dim3(256), lds, st, a, n_groups);
    else hipLaunchKernelGGL((gemm_prefill_persistent<2, false>), dim3(pgrid), dim3(256), lds, st, a, n_groups);
  } else if (d->n_w == 2) {
    if (a.lrq) hipLaunchKernelGGL((gemm_prefill_kernel<2, true, 64>), grid, dim3(256), lds, st, a);
    else hipLaunchKernelGGL((gemm_prefill_kernel<2, false, 64>), grid, dim3(256), lds, st, a);
  } else {
    if (a.lrq) hipLaunchKernelGGL((gemm_prefill_kernel<1, true, 64>), grid, dim3(256), lds, st, a);
    else hipLaunchKernelGGL((gemm_prefill_kernel<1, false, 64>), grid, dim3(256), lds, st, a);
  }
  return hip_status(hipGetLastError(), "gemm_prefill_kernel launch");
}

}  // namespace milo
