// Inputs of the adaptive compensator rank policy and the policy itself.
//
// [talk] = "MiLo: Efficient Quantized MoE Inference with Mixture of Low-Rank
// Compensators" (MLSys 2025 talk write-up), MiLo Algorithm, "Mixture of
// Low-Rank Compensators and Adaptive Rank Selection": higher ranks for dense
// (always-activated) parts, for frequently activated experts, and for weights
// with a higher kurtosis.
//
// * weight kurtosis on the GPU: two streaming passes over every matrix
//   (mean; then central second and fourth moments), float64 accumulation,
//   per-block partial sums added in block order by a one-block finisher --
//   deterministic, HBM-bound;
// * routed pairs per expert accumulated on the GPU from routing offsets;
// * the rank apportionment (host): score = frequency (1 for dense parts) x
//   kurtosis / 3, largest-remainder apportionment of a rank budget in steps
//   with per-matrix caps, ties to the lower index; the score sum runs left to
//   right so the integers are reproducible.
#include <math.h>

#include "milo_internal.hpp"

namespace milo {

constexpr int kMomThreads = 256;
constexpr int kMomMaxBlocks = 256;     // partial-sum blocks per matrix

__device__ __forceinline__ double block_sum(double v, double* red) {
  const int t = threadIdx.x;
  red[t] = v;
  __syncthreads();
  for (int w = kMomThreads / 2; w >= 1; w >>= 1) {
    if (t < w) red[t] += red[t + w];
    __syncthreads();
  }
  const double s = red[0];
  __syncthreads();
  return s;
}

// Sums over elements [e0, e1) of one matrix for this thread: PASS 0 sum of
// w - mu; PASS 1 sums of (w - mu)^2 and (w - mu)^4.  16-byte non-temporal
// loads (each weight is read once per pass), four in flight; e0 and the
// chunk are multiples of 4.  A thread adds its elements in ascending order.
template <int PASS>
__device__ __forceinline__ void moments_sums(const float* __restrict__ wm, int64_t e0, int64_t e1, double mu,
                                             double& s1, double& s2) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  double a1 = 0.0, a2 = 0.0;
  auto add = [&](double x) {
    const double d = x - mu;
    if (PASS) {
      const double d2 = d * d;
      a1 += d2;
      a2 += d2 * d2;
    } else {
      a1 += d;
    }
  };
  const int64_t step = 4 * (int64_t)kMomThreads;
  int64_t i = e0 + 4 * (int64_t)threadIdx.x;
  for (; i + 3 * step + 3 < e1; i += 4 * step) {
    f32x4_t q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) q[u] = __builtin_nontemporal_load((const f32x4_t*)(wm + i + u * step));
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int k = 0; k < 4; ++k) add((double)q[u][k]);
  }
  for (; i < e1; i += step) {
    if (i + 3 < e1) {
      const f32x4_t q = __builtin_nontemporal_load((const f32x4_t*)(wm + i));
#pragma unroll
      for (int k = 0; k < 4; ++k) add((double)q[k]);
    } else {
      for (int64_t k = i; k < e1; ++k) add((double)wm[k]);
    }
  }
  s1 = a1;
  s2 = a2;
}

// pass 0: sum of w;  pass 1: sum of (w - mean)^2 and (w - mean)^4.
// Block (b, m) covers elements [b chunk, (b + 1) chunk) of matrix m.
__global__ void __launch_bounds__(kMomThreads) moments_kernel(const float* __restrict__ W, int64_t elems,
                                                              int64_t chunk, int pass,
                                                              const double* __restrict__ mean,
                                                              double* __restrict__ part) {
  __shared__ double red[kMomThreads];
  const int m = blockIdx.y, b = blockIdx.x, nb = gridDim.x;
  const float* wm = W + (size_t)m * elems;
  const int64_t e0 = (int64_t)b * chunk;
  const int64_t e1 = e0 + chunk < elems ? e0 + chunk : elems;
  double s1 = 0.0, s2 = 0.0;
  if (pass) moments_sums<1>(wm, e0, e1, mean[m], s1, s2);
  else moments_sums<0>(wm, e0, e1, 0.0, s1, s2);
  const double t1 = block_sum(s1, red);
  const double t2 = pass ? block_sum(s2, red) : 0.0;
  if (threadIdx.x == 0) {
    part[((size_t)m * nb + b) * 2] = t1;
    part[((size_t)m * nb + b) * 2 + 1] = t2;
  }
}

// Adds the partial sums of each matrix in block order: pass 0 -> mean,
// pass 1 -> kurtosis n sum d^4 / (sum d^2)^2 (0 when there is no spread).
__global__ void __launch_bounds__(64) moments_finish_kernel(const double* __restrict__ part, int nb,
                                                            int64_t elems, int count, int pass,
                                                            double* __restrict__ mean,
                                                            double* __restrict__ kurt) {
  for (int m = blockIdx.x * blockDim.x + threadIdx.x; m < count; m += gridDim.x * blockDim.x) {
    // partials added in block order; eight blocks' loads in flight
    double a = 0.0, c = 0.0;
    const double* pm = part + (size_t)m * nb * 2;
    for (int b0 = 0; b0 < nb; b0 += 8) {
      double pa[8], pc[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        pa[u] = b0 + u < nb ? pm[(b0 + u) * 2] : 0.0;
        pc[u] = b0 + u < nb ? pm[(b0 + u) * 2 + 1] : 0.0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (b0 + u < nb) {
          a += pa[u];
          c += pc[u];
        }
      }
    }
    if (pass == 0) {
      mean[m] = a / (double)elems;
    } else {
      kurt[m] = a > 0.0 ? (double)elems * c / (a * a) : 0.0;
    }
  }
}

__global__ void __launch_bounds__(256) expert_counts_kernel(const int32_t* __restrict__ offsets, int E,
                                                            int64_t* __restrict__ counts) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) counts[e] += offsets[e + 1] - offsets[e];
}

static int moment_blocks(int64_t count) {
  int64_t b = 2048 / (count > 0 ? count : 1);
  return (int)(b < 1 ? 1 : (b > kMomMaxBlocks ? kMomMaxBlocks : b));
}

size_t kurtosis_workspace_bytes(int64_t count) {
  return ((size_t)count * kMomMaxBlocks * 2 + (size_t)count) * sizeof(double);
}

int32_t launch_kurtosis(const float* W, int64_t count, int64_t elems, double* kurt, double* mean_out,
                        char* ws, hipStream_t st) {
  const int nb = moment_blocks(count);
  int64_t chunk = (elems + nb - 1) / nb;
  chunk = (chunk + 3) / 4 * 4;
  double* part = (double*)ws;
  double* mean = mean_out ? mean_out : part + (size_t)count * kMomMaxBlocks * 2;
  const dim3 grid(nb, (unsigned)count);
  const int fin = (int)((count + 63) / 64);
  hipLaunchKernelGGL(moments_kernel, grid, dim3(kMomThreads), 0, st, W, elems, chunk, 0, mean, part);
  hipLaunchKernelGGL(moments_finish_kernel, dim3(fin), dim3(64), 0, st, part, nb, elems, (int)count, 0, mean,
                     kurt);
  hipLaunchKernelGGL(moments_kernel, grid, dim3(kMomThreads), 0, st, W, elems, chunk, 1, mean, part);
  hipLaunchKernelGGL(moments_finish_kernel, dim3(fin), dim3(64), 0, st, part, nb, elems, (int)count, 1, mean,
                     kurt);
  return hip_status(hipGetLastError(), "kurtosis launches");
}

int32_t launch_expert_counts(const int32_t* offsets, int E, int64_t* counts, hipStream_t st) {
  hipLaunchKernelGGL(expert_counts_kernel, dim3(1), dim3(256), 0, st, offsets, E, counts);
  return hip_status(hipGetLastError(), "expert_counts_kernel launch");
}

// ---------------------------------------------------------------- host policy

void rank_policy_host(const double* kurt, const double* freq, const int32_t* dense, int n, int total_rank,
                      int r_min, int r_max, int step, int32_t* ranks) {
  const int units = total_rank / step, lo = r_min / step, hi = r_max / step;
  double* target = new double[n];
  int* u = new int[n];
  double ssum = 0.0;
  for (int i = 0; i < n; ++i) {
    target[i] = ((dense[i] ? 1.0 : freq[i]) * kurt[i]) / 3.0;   // score first
    ssum += target[i];
  }
  for (int i = 0; i < n; ++i) target[i] = ssum > 0.0 ? (double)units * target[i] / ssum : (double)units / n;
  long left = units;
  for (int i = 0; i < n; ++i) {
    int v = (int)floor(target[i]);
    v = v < lo ? lo : (v > hi ? hi : v);
    u[i] = v;
    left -= v;
  }
  while (left > 0) {
    int best = -1;
    for (int i = 0; i < n; ++i)
      if (u[i] < hi && (best < 0 || target[i] - u[i] > target[best] - u[best])) best = i;
    if (best < 0) break;
    ++u[best];
    --left;
  }
  while (left < 0) {
    int best = -1;
    for (int i = 0; i < n; ++i)
      if (u[i] > lo && (best < 0 || target[i] - u[i] < target[best] - u[best])) best = i;
    if (best < 0) break;
    --u[best];
    ++left;
  }
  for (int i = 0; i < n; ++i) ranks[i] = u[i] * step;
  delete[] target;
  delete[] u;
}

}  // namespace milo
