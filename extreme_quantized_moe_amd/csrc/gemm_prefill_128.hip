// 128-row tile launches of the matrix-core (prefill) path.  A translation
// unit of their own so that the build can give them the max-ILP instruction
// scheduler (measured on the Mixtral-shaped prefill layer: gate/up 1.912 ->
// 1.870 ms, down 1.026 -> 1.009 ms; the 64-row kernels spill registers under
// it and keep the default scheduler).  Kernels in gemm_prefill_tiles.hpp.
#include "gemm_prefill_tiles.hpp"

namespace milo {

int32_t launch_gemm_prefill_128(const GemmArgs& a, int n_w, dim3 grid, hipStream_t st) {
  const size_t lds = prefill_lds(128) > prefill_lds_128 ? prefill_lds(128) : prefill_lds_128;
  if (n_w == 2) {
    if (a.lrq) hipLaunchKernelGGL((gemm_prefill_kernel<2, true, 128>), grid, dim3(256), lds, st, a);
    else hipLaunchKernelGGL((gemm_prefill_kernel<2, false, 128>), grid, dim3(256), lds, st, a);
  } else {
    if (a.lrq) hipLaunchKernelGGL((gemm_prefill_kernel<1, true, 128>), grid, dim3(256), lds, st, a);
    else hipLaunchKernelGGL((gemm_prefill_kernel<1, false, 128>), grid, dim3(256), lds, st, a);
  }
  return hip_status(hipGetLastError(), "gemm_prefill_kernel launch");
}

}  // namespace milo
