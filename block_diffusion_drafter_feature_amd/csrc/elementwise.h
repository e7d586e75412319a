// Row-wise kernels of the drafter: RMSNorm (optionally gathering the embedding rows
// first), the dynamic short conv's apply step.  One work-group per row; fixed-order reductions.
#pragma once

#include "common.h"

namespace dflash {

// u = x / sqrt(mean(x^2) + eps) * g.  Writes u rounded to T (out_t) and/or in fp32 (out_f).
// One work-group per row; each thread owns 4-float groups c = tid, tid + 256, ... and issues
// all of its row loads before reducing (d <= 256 * 4 * 16 per row in one pass of registers).
// With emb != nullptr the row is first gathered: x[m] = E[ids[m]] widened to fp32 (and
// stored to x), then normalised -- the embedding step and the first norm in one pass.
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(float* __restrict__ x, const T* __restrict__ g, int d,
                                                      float eps, T* __restrict__ out_t, float* __restrict__ out_f,
                                                      const T* __restrict__ emb = nullptr,
                                                      const int32_t* __restrict__ ids = nullptr) {
  constexpr int MAXV = 16;
  __shared__ float red[8];
  const int m = blockIdx.x;
  f32x4_t* const xw = reinterpret_cast<f32x4_t*>(x + static_cast<size_t>(m) * d);
  const f32x4_t* xr = xw;
  const T* er = emb ? emb + static_cast<size_t>(ids[m]) * d : nullptr;
  auto src = [&](int c) {
    if (!er) return xr[c];
    const f32x4_t t{to_f<T>(er[4 * c]), to_f<T>(er[4 * c + 1]), to_f<T>(er[4 * c + 2]), to_f<T>(er[4 * c + 3])};
    xw[c] = t;
    return t;
  };
  const int nv = d >> 2;
  f32x4_t v[MAXV];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = threadIdx.x + 256 * i;
    v[i] = c < nv ? src(c) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int i = 0; i < MAXV; ++i) ss += v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3];
  for (int c = threadIdx.x + 256 * MAXV; c < nv; c += 256) {
    const f32x4_t t = src(c);
    ss += t[0] * t[0] + t[1] * t[1] + t[2] * t[2] + t[3] * t[3];
  }
  ss = block_sum(ss, red);
  const float inv = 1.f / sqrtf(ss / d + eps);
  auto emit = [&](int c, const f32x4_t& t) {
    float u[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = t[e] * inv * to_f<T>(g[4 * c + e]);
    if (out_t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) out_t[static_cast<size_t>(m) * d + 4 * c + e] = from_f<T>(u[e]);
    }
    if (out_f) *reinterpret_cast<f32x4_t*>(out_f + static_cast<size_t>(m) * d + 4 * c) = f32x4_t{u[0], u[1], u[2], u[3]};
  };
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < nv) emit(c, v[i]);
  }
  for (int c = threadIdx.x + 256 * MAXV; c < nv; c += 256) emit(c, xr[c]);
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
