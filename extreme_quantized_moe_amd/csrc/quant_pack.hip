// Offline weight preparation on the GPU: RTN int3 quantization and the
// layout-v1 repack.
//
// [talk] = "MiLo: Efficient Quantized MoE Inference with Mixture of Low-Rank
// Compensators" (MLSys 2025 talk write-up).  Background: RTN is the simplest
// calibration-free quantizer; MiLo Algorithm / Key Findings: int3 weights
// with an asymmetric zero point; MiLo Kernel, "Bit Packing": 32 three-bit
// values in three 32-bit words, no bit wasted.
#include "milo_internal.hpp"

namespace milo {

// float64 -> float16 bits, round to nearest even, computed directly from the
// double (a float32 intermediate would round twice).
__device__ uint16_t f64_to_f16_rne(double x) {
  uint64_t b = (uint64_t)__double_as_longlong(x);
  uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  int ex = (int)((b >> 52) & 0x7FF);
  uint64_t mant = b & 0xFFFFFFFFFFFFFull;
  if (ex == 0x7FF) return sign | 0x7C00u | (mant ? 0x200u : 0u);
  int e = ex - 1023;
  if (ex == 0) return sign;                  // float64 subnormals underflow
  if (e > 15) return sign | 0x7C00u;
  if (e >= -14) {                            // normal float16
    uint64_t m = mant >> 42, rem = mant & ((1ull << 42) - 1), half = 1ull << 41;
    uint32_t h = ((uint32_t)(e + 15) << 10) | (uint32_t)m;
    if (rem > half || (rem == half && (m & 1))) h += 1;  // may carry into exponent
    return (uint16_t)(sign | h);
  }
  if (e < -25) return sign;
  uint64_t full = (1ull << 52) | mant;       // value = full * 2^(e-52)
  int shift = 52 - (e + 24);                 // 43..53: in units of 2^-24
  uint64_t q = full >> shift, rem = full & ((1ull << shift) - 1), half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) q += 1;
  return (uint16_t)(sign | q);
}

__device__ __forceinline__ double f16_bits_to_f64(uint16_t h) {
  return (double)(float)__builtin_bit_cast(_Float16, h);
}

// One wave per (row, group): lane = column inside the group (group <= 64;
// lanes past the group take part in the min/max with the group's first value).
__global__ void __launch_bounds__(256) quantize_kernel(const float* __restrict__ W, int64_t rows,
                                                       int64_t K, int group,
                                                       uint8_t* __restrict__ codes,
                                                       uint16_t* __restrict__ scale,
                                                       uint16_t* __restrict__ zero) {
  const int lane = threadIdx.x & 63;
  const int64_t groups = K / group;
  const int64_t total = rows * groups;
  const int64_t wave0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  const bool in = lane < group;
  for (int64_t gi = wave0; gi < total; gi += nwaves) {
    const int64_t r = gi / groups, g = gi - r * groups;
    const int64_t idx = r * K + g * group + (in ? lane : 0);
    const float w = W[idx];
    float lo = w, hi = w;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      lo = fminf(lo, __shfl_xor(lo, o));
      hi = fmaxf(hi, __shfl_xor(hi, o));
    }
    uint16_t sb = f64_to_f16_rne(((double)hi - (double)lo) / 7.0);
    if ((sb & 0x7FFFu) == 0) sb = 0x3C00u;  // s == 0 -> 1
    const double s = f16_bits_to_f64(sb);
    double zr = -(double)lo / s;
    zr = fmin(fmax(zr, -65504.0), 65504.0);
    const uint16_t zb = f64_to_f16_rne(zr);
    const double z = f16_bits_to_f64(zb);
    double q = rint((double)w / s + z);
    q = fmin(fmax(q, 0.0), 7.0);
    if (in) codes[idx] = (uint8_t)q;
    if (lane == 0) {
      scale[r * groups + g] = sb;
      zero[r * groups + g] = zb;
    }
  }
}

// One thread per triplet (tile, lane L, row group i).
__global__ void __launch_bounds__(256) pack_kernel(const uint8_t* __restrict__ codes,
                                                   const uint16_t* __restrict__ scale,
                                                   const uint16_t* __restrict__ zero,
                                                   int64_t rows, int64_t K,
                                                   uint32_t* __restrict__ packed,
                                                   uint32_t* __restrict__ sz) {
  const int64_t kblocks = K / kTileK;
  const int64_t ntrip = (rows / kTileRows) * kblocks * 256;
  for (int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; tid < ntrip;
       tid += (int64_t)gridDim.x * blockDim.x) {
    const int64_t tile = tid >> 8;
    const int L = (int)((tid >> 2) & 63);
    const int i = (int)(tid & 3);
    const int64_t rt = tile / kblocks, kb = tile - rt * kblocks;
    const int64_t r = rt * kTileRows + 16 * i + (L & 15);
    const int kq = L >> 4;
    uint32_t word[3] = {0u, 0u, 0u};
    const uint8_t* rowp = codes + r * K + kb * kTileK + 8 * kq;
#pragma unroll
    for (int step = 0; step < 4; ++step) {
      // codes c = 8 step + t, t = 0..7, at column 128 kb + 32 step + 8 kq + t
      uint64_t eight = *(const uint64_t*)(rowp + 32 * step);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t q = (uint32_t)((eight >> (8 * t)) & 7u);
        const int c = 8 * step + t, pi = c >> 1, h = c & 1;
        if (pi < 15) {
          word[pi / 5] |= q << (16 * h + 1 + 3 * (pi % 5));
        } else {
#pragma unroll
          for (int b = 0; b < 3; ++b) word[b] |= ((q >> b) & 1u) << (16 * h);
        }
      }
    }
    uint32_t* tp = packed + tile * kTileWords + 4 * L + i;
    tp[0] = word[0];
    tp[256] = word[1];
    tp[512] = word[2];
    if (kq < 2) {  // lanes of K-quarters 0 and 1 write the row's two group words
      const int64_t gg = 2 * kb + kq;
      const int64_t groups = K / kGroup;
      sz[tile * kTileSzWords + 8 * (L & 15) + 2 * i + kq] =
          (uint32_t)scale[r * groups + gg] | ((uint32_t)zero[r * groups + gg] << 16);
    }
  }
}

// Sum over the 64 lanes of a wave; the xor butterfly adds the same pairs in
// every lane, so all lanes hold the identical sum.
// DPP move of a 32-bit value / a double (both halves) inside rows of 16
// lanes; CTRL is a permutation that stays inside the row, so every lane has
// a source.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Sum over the 8 lanes of an aligned lane group, the same value in all of
// them, in a fixed order: swap neighbours, swap pairs, half-row mirror (each
// step adds two equal partial sums in either order).
__device__ __forceinline__ double sum8(double v) {
  v += dpp_f64<0xB1>(v);    // quad_perm [1, 0, 3, 2]
  v += dpp_f64<0x4E>(v);    // quad_perm [2, 3, 0, 1]
  v += dpp_f64<0x141>(v);   // row_half_mirror
  return v;
}
__device__ __forceinline__ float min8(float v) {
  v = fminf(v, dpp_f32<0xB1>(v));
  v = fminf(v, dpp_f32<0x4E>(v));
  return fminf(v, dpp_f32<0x141>(v));
}
__device__ __forceinline__ float max8(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  return fmaxf(v, dpp_f32<0x141>(v));
}

// Code of a weight at zero point z given ws = w / s (the division is taken
// once per weight: codes depend on w / s + z only).
__device__ __forceinline__ double code_at(double ws, double z) { return fmin(fmax(rint(ws + z), 0.0), 7.0); }

// HQQ-style zero-point optimization of each group of 64, float64: start from
// the RTN scale and zero point; each iteration quantizes with the current
// zero point z, takes the generalized soft threshold of the error, updates
// z = mean(q - (w - W_e) / s), beta *= kappa; the fp16 candidate f16(z) is
// scored by the group's mean absolute error with codes chosen at it, and the
// best candidate (the RTN zero point first) is kept.
//
// Eight lanes per group, eight consecutive weights per lane (a wave holds
// eight groups; 32-byte loads, 8-byte code stores); group sums are the lane's
// sum of its eight terms in order, then the 8-lane tree above.
//
// The threshold is zero unless |x|^(2-p) > 1 / beta, so for |x| at most half
// of beta_last^(-1 / (2 - p)) (beta_last the largest beta used; beta never
// decreases) W_e is exactly 0 and the power is skipped; then
// (w - W_e) / s = w / s exactly.  For weights of the usual magnitude that is
// every weight.
__global__ void __launch_bounds__(256) hqq_kernel(const float* __restrict__ W, int64_t rows, int64_t K,
                                                  int iters, double p, double beta, double kappa,
                                                  uint8_t* __restrict__ codes, uint16_t* __restrict__ scale,
                                                  uint16_t* __restrict__ zero) {
  const int l8 = threadIdx.x & 7;
  const int64_t groups = K / kGroup;
  const int64_t total = rows * groups;
  const int64_t g0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 3;
  const int64_t ng = ((int64_t)gridDim.x * blockDim.x) >> 3;
  const double skip = iters > 0 ? 0.5 * pow(beta * pow(kappa, (double)(iters - 1)), -1.0 / (2.0 - p)) : 0.0;
  // the loop runs the same number of times in all 8 lanes of a group
  for (int64_t gi = g0; gi < total; gi += ng) {
    const int64_t r = gi / groups, g = gi - r * groups;
    const int64_t idx = r * K + g * kGroup + 8 * l8;
    const float4 a0 = *(const float4*)(W + idx);
    const float4 a1 = *(const float4*)(W + idx + 4);
    const float wf[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    float lo = wf[0], hi = wf[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) {
      lo = fminf(lo, wf[j]);
      hi = fmaxf(hi, wf[j]);
    }
    lo = min8(lo);
    hi = max8(hi);
    uint16_t sb = f64_to_f16_rne(((double)hi - (double)lo) / 7.0);
    if ((sb & 0x7FFFu) == 0) sb = 0x3C00u;
    const double s = f16_bits_to_f64(sb);
    const uint16_t z0b = f64_to_f16_rne(fmin(fmax(-(double)lo / s, -65504.0), 65504.0));
    double w[8], ws[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      w[j] = (double)wf[j];
      ws[j] = w[j] / s;
    }
    double z = f16_bits_to_f64(z0b);
    uint16_t best_b = z0b;
    double best_z = z;
    double best_err = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j) best_err += fabs(w[j] - (code_at(ws[j], z) - z) * s);
    best_err = sum8(best_err);
    double b = beta;
    for (int it = 0; it < iters; ++it) {
      double acc = 0.0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const double q = code_at(ws[j], z);
        const double x = w[j] - (q - z) * s;
        const double ax = fabs(x);
        double u = ws[j];                  // (w - W_e) / s with W_e = 0
        if (ax > skip) {
          const double t = ax - pow(ax, p - 1.0) / b;
          if (t > 0.0) u = (w[j] - copysign(t, x)) / s;
        }
        acc += q - u;
      }
      z = sum8(acc) / (double)kGroup;
      b *= kappa;
      const uint16_t zb = f64_to_f16_rne(fmin(fmax(z, -65504.0), 65504.0));
      const double zc = f16_bits_to_f64(zb);
      double err = 0.0;
#pragma unroll
      for (int j = 0; j < 8; ++j) err += fabs(w[j] - (code_at(ws[j], zc) - zc) * s);
      err = sum8(err);
      if (err < best_err) {
        best_err = err;
        best_z = zc;
        best_b = zb;
      }
    }
    uint32_t c0 = 0, c1 = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c0 |= (uint32_t)code_at(ws[j], best_z) << (8 * j);
      c1 |= (uint32_t)code_at(ws[j + 4], best_z) << (8 * j);
    }
    *(uint2*)(codes + idx) = make_uint2(c0, c1);
    if (l8 == 0) {
      scale[r * groups + g] = sb;
      zero[r * groups + g] = best_b;
    }
  }
}

// Set the bits of code c (value q) of a triplet, layout v1 bit assignment.
__device__ __forceinline__ void put_code(uint32_t (&word)[3], int c, uint32_t q) {
  const int pi = c >> 1, h = c & 1;
  if (pi < 15) {
    word[pi / 5] |= q << (16 * h + 1 + 3 * (pi % 5));
  } else {
#pragma unroll
    for (int b = 0; b < 3; ++b) word[b] |= ((q >> b) & 1u) << (16 * h);
  }
}

constexpr uint32_t kPadSz = 0x00003C00u;   // scale 1.0, zero 0.0

// V factor of an int3 compensator: one thread per (rank row j, triplet tau);
// the threads of triplets kq = 0 and 1 of each 128-wide block also write the
// row's two group words.
__global__ void __launch_bounds__(256) pack_lr_v_kernel(const uint8_t* __restrict__ codes,
                                                        const uint16_t* __restrict__ scale,
                                                        const uint16_t* __restrict__ zero,
                                                        int rank, int max_rank, int64_t K,
                                                        uint32_t* __restrict__ vq,
                                                        uint32_t* __restrict__ vsz) {
  const int64_t T32 = K / 32, groups = K / kGroup;
  const int64_t n = (int64_t)max_rank * T32;
  for (int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; tid < n;
       tid += (int64_t)gridDim.x * blockDim.x) {
    const int64_t j = tid / T32, tau = tid - j * T32;
    const int64_t kb = tau >> 2;
    const int kq = (int)(tau & 3);
    uint32_t word[3] = {0u, 0u, 0u};
    if (j < rank) {
      const uint8_t* rowp = codes + j * K + kb * kTileK + 8 * kq;
#pragma unroll
      for (int c = 0; c < 32; ++c) put_code(word, c, rowp[32 * (c >> 3) + (c & 7)] & 7u);
    }
    vq[3 * tid] = word[0];
    vq[3 * tid + 1] = word[1];
    vq[3 * tid + 2] = word[2];
    if (kq < 2) {
      const int64_t gg = 2 * kb + kq;
      vsz[j * groups + gg] =
          j < rank ? ((uint32_t)scale[j * groups + gg] | ((uint32_t)zero[j * groups + gg] << 16)) : kPadSz;
    }
  }
}

// U factor: one thread per (64-row x 32-rank tile, lane); the lanes of rank
// tile 0 also write their n-tile's scale/zero words.
__global__ void __launch_bounds__(256) pack_lr_u_kernel(const uint8_t* __restrict__ codes,
                                                        const uint16_t* __restrict__ scale,
                                                        const uint16_t* __restrict__ zero,
                                                        int64_t N, int rank, int R32,
                                                        uint32_t* __restrict__ uq,
                                                        uint32_t* __restrict__ usz) {
  const int JT = R32 / 32;
  const int64_t n_all = (N / kTileRows) * JT * 64;
  for (int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; tid < n_all;
       tid += (int64_t)gridDim.x * blockDim.x) {
    const int64_t tile = tid >> 6;
    const int L = (int)(tid & 63);
    const int64_t nt = tile / JT;
    const int jt = (int)(tile - nt * JT);
    uint32_t word[3] = {0u, 0u, 0u};
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      const int64_t n = 64 * nt + 16 * (c >> 3) + (L & 15);
      const int j = 32 * jt + 8 * (L >> 4) + (c & 7);
      if (j < rank) put_code(word, c, codes[n * rank + j] & 7u);
    }
    uint32_t* tp = uq + tile * 192 + L;
    tp[0] = word[0];
    tp[64] = word[1];
    tp[128] = word[2];
    if (jt == 0) {
      const int64_t n = 64 * nt + L;
      usz[64 * nt + 4 * (L & 15) + (L >> 4)] =
          rank > 0 ? ((uint32_t)scale[n] | ((uint32_t)zero[n] << 16)) : kPadSz;
    }
  }
}

static int grid_for(int64_t work, int per_block) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

int32_t launch_quantize(const float* W, int64_t rows, int64_t K, int group, uint8_t* codes,
                        uint16_t* scale, uint16_t* zero, hipStream_t st) {
  const int64_t waves = rows * (K / group);
  hipLaunchKernelGGL(quantize_kernel, dim3(grid_for(waves, 4)), dim3(256), 0, st, W, rows, K,
                     group, codes, scale, zero);
  return hip_status(hipGetLastError(), "quantize_kernel launch");
}

int32_t launch_pack(const uint8_t* codes, const uint16_t* scale, const uint16_t* zero,
                    int64_t rows, int64_t K, uint32_t* packed, uint32_t* sz, hipStream_t st) {
  const int64_t ntrip = (rows / kTileRows) * (K / kTileK) * 256;
  hipLaunchKernelGGL(pack_kernel, dim3(grid_for(ntrip, 256)), dim3(256), 0, st, codes, scale,
                     zero, rows, K, packed, sz);
  return hip_status(hipGetLastError(), "pack_kernel launch");
}

int32_t launch_pack_lr(const uint8_t* v_codes, const uint16_t* v_scale, const uint16_t* v_zero,
                       const uint8_t* u_codes, const uint16_t* u_scale, const uint16_t* u_zero,
                       int64_t N, int64_t K, int rank, int max_rank, uint32_t* vq, uint32_t* vsz,
                       uint32_t* uq, uint32_t* usz, hipStream_t st) {
  const int R32 = (max_rank + 31) / 32 * 32;
  const int64_t nv = (int64_t)max_rank * (K / 32);
  hipLaunchKernelGGL(pack_lr_v_kernel, dim3(grid_for(nv, 256)), dim3(256), 0, st, v_codes, v_scale,
                     v_zero, rank, max_rank, K, vq, vsz);
  int32_t rc = hip_status(hipGetLastError(), "pack_lr_v_kernel launch");
  if (rc != MILO_OK) return rc;
  const int64_t nu = (N / kTileRows) * (R32 / 32) * 64;
  hipLaunchKernelGGL(pack_lr_u_kernel, dim3(grid_for(nu, 256)), dim3(256), 0, st, u_codes, u_scale,
                     u_zero, N, rank, R32, uq, usz);
  return hip_status(hipGetLastError(), "pack_lr_u_kernel launch");
}

int32_t launch_hqq(const float* W, int64_t rows, int64_t K, int iters, double p, double beta, double kappa,
                   uint8_t* codes, uint16_t* scale, uint16_t* zero, hipStream_t st) {
  const int64_t groups = rows * (K / kGroup);      // 32 groups per 256-thread block
  hipLaunchKernelGGL(hqq_kernel, dim3(grid_for(groups, 32)), dim3(256), 0, st, W, rows, K, iters, p, beta, kappa,
                     codes, scale, zero);
  return hip_status(hipGetLastError(), "hqq_kernel launch");
}

}  // namespace milo
