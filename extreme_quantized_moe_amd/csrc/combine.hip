// Weighted combine of a token's slot outputs: out[t] = sum_j y[t*slots + j]
// in slot order (float32), rounded once to float16.
// [talk] = "MiLo: Efficient Quantized MoE Inference with Mixture of Low-Rank
// Compensators" (MLSys 2025 talk write-up), Background: a token's output
// combines the outputs of the experts it activates.
#include "milo_internal.hpp"

namespace milo {

// MS bounds the slots per token (the slot loop is unrolled to it: the kernel
// runs cold from the instruction cache, so top-2 routing gets a short one);
// the element index is 32-bit (the launcher checks that T * H / 4 fits).
template <int MS>
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ y, int T, int slots,
                                                      int H, uint16_t* __restrict__ out) {
  const int hq = H >> 2;
  const int total = T * hq;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
    const int t = i / hq;
    const int h4 = i - t * hq;
    const float4* src = (const float4*)(y + (size_t)t * slots * H) + h4;
    float4 v[MS];                         // all slot loads issued before the sum
#pragma unroll
    for (int j = 0; j < MS; ++j)
      if (j < slots) v[j] = src[(size_t)j * hq];
    float4 acc = v[0];
#pragma unroll
    for (int j = 1; j < MS; ++j)
      if (j < slots) {
        acc.x += v[j].x; acc.y += v[j].y; acc.z += v[j].z; acc.w += v[j].w;
      }
    uint2 o;
    o.x = (uint32_t)float_to_half_bits(acc.x) | ((uint32_t)float_to_half_bits(acc.y) << 16);
    o.y = (uint32_t)float_to_half_bits(acc.z) | ((uint32_t)float_to_half_bits(acc.w) << 16);
    ((uint2*)(out + (size_t)t * H))[h4] = o;
  }
}

int32_t launch_combine(const float* y, int T, int slots, int H, uint16_t* out, hipStream_t st) {
  const int64_t work = (int64_t)T * (H / 4);
  if (work > 0x7F000000) {   // headroom for the grid-stride step
    set_error("T * H / 4 = %lld elements exceed the combine kernel's 32-bit index", (long long)work);
    return MILO_ERR_SHAPE;
  }
  int64_t g = (work + 255) / 256;
  if (g > 16384) g = 16384;
  if (slots <= 4) hipLaunchKernelGGL(combine_kernel<4>, dim3((int)g), dim3(256), 0, st, y, T, slots, H, out);
  else hipLaunchKernelGGL(combine_kernel<16>, dim3((int)g), dim3(256), 0, st, y, T, slots, H, out);
  return hip_status(hipGetLastError(), "combine_kernel launch");
}

}  // namespace milo
