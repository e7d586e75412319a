// Row-wise kernels of the drafter: RMSNorm (optionally gathering the embedding rows
// first), the calibration MLP's input rows, rounding fp32 rows to the weights' type, FP8
// weight quantization.  One work-group per row; fixed-order reductions.
#pragma once

#include "common.h"

namespace dflash {

// 4 consecutive elements of T as floats / stored from floats (8-byte bf16 or 16-byte fp32
// accesses; p is 4-element aligned)
template <typename T>
__device__ __forceinline__ f32x4_t load4(const T* p) {
  if constexpr (sizeof(T) == 4) {
    return *reinterpret_cast<const f32x4_t*>(p);
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    return f32x4_t{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
                   __uint_as_float(v.y & 0xffff0000u)};
  }
}
template <typename T>
__device__ __forceinline__ void store4(T* p, const float (&u)[4]) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<f32x4_t*>(p) = f32x4_t{u[0], u[1], u[2], u[3]};
  } else {
    uint2 v;
    v.x = static_cast<uint32_t>(from_f<T>(u[0])) | (static_cast<uint32_t>(from_f<T>(u[1])) << 16);
    v.y = static_cast<uint32_t>(from_f<T>(u[2])) | (static_cast<uint32_t>(from_f<T>(u[3])) << 16);
    *reinterpret_cast<uint2*>(p) = v;
  }
}

// u = x / sqrt(mean(x^2) + eps) * g.  Writes u rounded to T (out_t) and/or in fp32 (out_f).
// One work-group per row; each thread owns 4-float groups c = tid, tid + 256, ... and issues
// all of its row loads, and the loads of its gains, before reducing (d <= 256 * 4 * MAXV per
// row in one pass of registers), so the row costs one memory round trip before the stores.
// MAXV = 4 (d <= 4096) keeps the register count low enough for more rows in flight per
// compute unit; the sums are the same for every MAXV (the extra groups add zeros).
// With emb != nullptr the row is first gathered: x[m] = E[ids[m]] widened to fp32 (and
// stored to x), then normalised -- the embedding step and the first norm in one pass.
template <typename T, int MAXV = 16>
__global__ __launch_bounds__(256) void rmsnorm_kernel(float* __restrict__ x, const T* __restrict__ g, int d,
                                                      float eps, T* __restrict__ out_t, float* __restrict__ out_f,
                                                      const T* __restrict__ emb = nullptr,
                                                      const int32_t* __restrict__ ids = nullptr) {
  __shared__ float red[8];
  const int m = blockIdx.x;
  f32x4_t* const xw = reinterpret_cast<f32x4_t*>(x + static_cast<size_t>(m) * d);
  const f32x4_t* xr = xw;
  const T* er = emb ? emb + static_cast<size_t>(ids[m]) * d : nullptr;
  auto src = [&](int c) {
    if (!er) return xr[c];
    const f32x4_t t = load4<T>(er + 4 * c);
    xw[c] = t;
    return t;
  };
  const int nv = d >> 2;
  f32x4_t v[MAXV], gv[MAXV];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = threadIdx.x + 256 * i;
    v[i] = c < nv ? src(c) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    gv[i] = c < nv ? load4<T>(g + 4 * c) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int i = 0; i < MAXV; ++i) ss += v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3];
  for (int c = threadIdx.x + 256 * MAXV; c < nv; c += 256) {
    const f32x4_t t = src(c);
    ss += t[0] * t[0] + t[1] * t[1] + t[2] * t[2] + t[3] * t[3];
  }
  ss = block_sum(ss, red);
  const float inv = 1.f / sqrtf(ss / d + eps);
  auto emit = [&](int c, const f32x4_t& t, const f32x4_t& gg) {
    float u[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = t[e] * inv * gg[e];
    if (out_t) store4<T>(out_t + static_cast<size_t>(m) * d + 4 * c, u);
    if (out_f) *reinterpret_cast<f32x4_t*>(out_f + static_cast<size_t>(m) * d + 4 * c) = f32x4_t{u[0], u[1], u[2], u[3]};
  };
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < nv) emit(c, v[i], gv[i]);
  }
  for (int c = threadIdx.x + 256 * MAXV; c < nv; c += 256) emit(c, xr[c], load4<T>(g + 4 * c));
}

template <typename T>
inline void launch_rmsnorm(int rows, hipStream_t s, float* x, const T* g, int d, float eps, T* out_t, float* out_f,
                           const T* emb = nullptr, const int32_t* ids = nullptr) {
  if (d <= 256 * 4 * 4)
    rmsnorm_kernel<T, 4><<<rows, 256, 0, s>>>(x, g, d, eps, out_t, out_f, emb, ids);
  else
    rmsnorm_kernel<T><<<rows, 256, 0, s>>>(x, g, d, eps, out_t, out_f, emb, ids);
}

// ------------------------------------------------------------------ bonus calibration input

// Row m of the calibration MLP's input: [E[bonus of m's sequence] ; xhat_m rounded to T].
// One work-group per row (16 rows per sequence).
template <typename T>
__global__ __launch_bounds__(256) void cal_input_kernel(const T* __restrict__ emb, const int32_t* __restrict__ bonus,
                                                        const float* __restrict__ xhat, int d, T* __restrict__ out) {
  const int m = blockIdx.x;
  const T* e = emb + static_cast<size_t>(bonus[m >> 4]) * d;
  const float* x = xhat + static_cast<size_t>(m) * d;
  T* o = out + static_cast<size_t>(m) * 2 * d;
  for (int j = threadIdx.x; j < d; j += 256) {
    o[j] = e[j];
    o[d + j] = from_f<T>(x[j]);
  }
}

// ------------------------------------------------------------------ rounding to T

// y = x rounded to T, 4 elements per thread (n a multiple of 4, both 4-element aligned):
// hands fp32 rows to the bf16 GEMM kernels, which read A only in the weights' type.
template <typename T>
__global__ __launch_bounds__(256) void round_to_kernel(const float* __restrict__ x, size_t n4, T* __restrict__ y) {
  for (size_t i = blockIdx.x * static_cast<size_t>(256) + threadIdx.x; i < n4; i += static_cast<size_t>(gridDim.x) * 256) {
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(x + 4 * i);
    const float u[4] = {v[0], v[1], v[2], v[3]};
    store4<T>(y + 4 * i, u);
  }
}

// ------------------------------------------------------------------ FP8 weight storage

// E4M3 code of the value nearest to x (ties to the even mantissa), magnitudes saturating
// at 448; zero encodes as 0.  Below 2^-6 the grid is the multiples of 2^-9 (code = the
// multiple, 8 being the smallest normal); above, 3 mantissa bits rounded from float32's
// 23, a carry moving into the exponent field.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t sign = __float_as_uint(x) >> 31;
  const float a = fminf(fabsf(x), 448.f);
  uint32_t code;
  if (a < 0.015625f) {
    code = static_cast<uint32_t>(rintf(a * 512.f));
  } else {
    const uint32_t b = __float_as_uint(a);
    const uint32_t e = (b >> 23) - 120u;          // biased E4M3 exponent, 1 .. 15
    const uint32_t keep = (b >> 20) & 7u, rem = b & 0xFFFFFu;
    const uint32_t up = (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) ? 1u : 0u;
    code = (e << 3) + keep + up;
    code = code > 0x7Eu ? 0x7Eu : code;
  }
  return code ? (code | (sign << 7)) : 0u;
}

// One row per work-group: row scale = max |w| / 448, codes of w / scale, then the scale
// and 12 zero bytes (row stride cols + 16 bytes).
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const bf16_t* __restrict__ w, int cols,
                                                           uint8_t* __restrict__ out) {
  __shared__ float red[4];
  const bf16_t* row = w + static_cast<size_t>(blockIdx.x) * cols;
  uint8_t* o = out + static_cast<size_t>(blockIdx.x) * (cols + 16);
  float amax = 0.f;
  for (int j = threadIdx.x; j < cols; j += 256) amax = fmaxf(amax, fabsf(bf2f(row[j])));
#pragma unroll
  for (int k = 32; k > 0; k >>= 1) amax = fmaxf(amax, __shfl_xor(amax, k, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float scale = amax / 448.f;
  for (int j = threadIdx.x; j < cols; j += 256)
    o[j] = scale > 0.f ? static_cast<uint8_t>(e4m3_code(bf2f(row[j]) / scale)) : uint8_t{0};
  if (threadIdx.x < 4)
    reinterpret_cast<float*>(o + cols)[threadIdx.x] = threadIdx.x == 0 ? scale : 0.f;
}

}  // namespace dflash
