// Row-wise kernels of the drafter: embedding gather, RMSNorm, the dynamic short
// conv's apply step.  One work-group per row; fixed-order reductions.
#pragma once

#include "common.h"

namespace dflash {

// x[m] = E[ids[m]] widened to fp32.
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const T* __restrict__ E, const int32_t* __restrict__ ids, int d,
                                                    float* __restrict__ x) {
  const int m = blockIdx.x;
  const T* e = E + static_cast<size_t>(ids[m]) * d;
  for (int k = threadIdx.x; k < d; k += blockDim.x) x[static_cast<size_t>(m) * d + k] = to_f<T>(e[k]);
}

// u = x / sqrt(mean(x^2) + eps) * g.  Writes u rounded to T (out_t) and/or in fp32 (out_f).
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x, const T* __restrict__ g, int d,
                                                      float eps, T* __restrict__ out_t, float* __restrict__ out_f) {
  __shared__ float red[8];
  const int m = blockIdx.x;
  const float* xr = x + static_cast<size_t>(m) * d;
  float ss = 0.f;
  for (int k = threadIdx.x; k < d; k += blockDim.x) ss += xr[k] * xr[k];
  ss = block_sum(ss, red);
  const float inv = 1.f / sqrtf(ss / d + eps);
  for (int k = threadIdx.x; k < d; k += blockDim.x) {
    const float u = xr[k] * inv * to_f<T>(g[k]);
    if (out_t) out_t[static_cast<size_t>(m) * d + k] = from_f<T>(u);
    if (out_f) out_f[static_cast<size_t>(m) * d + k] = u;
  }
}

// Dynamic short conv, apply step, for block rows m (row j = m % 16 of its block):
//   a = w0 + delta[m][c/16],  b = w1 + delta[m][d/16 + c/16]
//   y = u[m] + a * u[m] + b * u[m-1]     (u[m-1] = 0 on block row 0)
// mode 0: out_t[m] = y rounded to T (a GEMM operand);  mode 1: x[m] += y (residual).
template <typename T>
__global__ __launch_bounds__(256) void conv_apply_kernel(const float* __restrict__ u, const float* __restrict__ delta,
                                                         const T* __restrict__ w0, const T* __restrict__ w1, int d,
                                                         int mode, T* __restrict__ out_t, float* __restrict__ x) {
  const int m = blockIdx.x, j = m & 15, ng = d / 16;
  const float* ur = u + static_cast<size_t>(m) * d;
  const float* dr = delta + static_cast<size_t>(m) * 2 * ng;
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    const float a = to_f<T>(w0[c]) + dr[c >> 4];
    const float bb = to_f<T>(w1[c]) + dr[ng + (c >> 4)];
    const float prev = j > 0 ? ur[c - d] : 0.f;
    const float y = ur[c] + a * ur[c] + bb * prev;
    if (mode == 0) out_t[static_cast<size_t>(m) * d + c] = from_f<T>(y);
    else x[static_cast<size_t>(m) * d + c] += y;
  }
}

}  // namespace dflash
