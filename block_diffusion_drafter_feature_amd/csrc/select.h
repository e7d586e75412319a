// Selection kernels: top-16 over the vocabulary, greedy verification, the Path
// Selector's pair scores and path walk.  All reductions use the total order
// (value descending, index ascending), so results are unique and deterministic.
#pragma once

#include "common.h"
#include <limits.h>
#include <type_traits>

namespace dflash {

// ------------------------------------------------------------------ register top-16 lists

struct Top16 {
  float v[16];
  int i[16];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      v[k] = -INFINITY;
      i[k] = INT_MAX;
    }
  }
  __device__ __forceinline__ void cswap(int a, int b) {   // keep the better of (a, b) at a
    const bool sw = better(v[b], i[b], v[a], i[a]);
    const float tv = sw ? v[b] : v[a];
    const int ti = sw ? i[b] : i[a];
    v[b] = sw ? v[a] : v[b];
    i[b] = sw ? i[a] : i[b];
    v[a] = tv;
    i[a] = ti;
  }
  // insert one candidate into the sorted list
  __device__ __forceinline__ void push(float x, int id) {
    if (!better(x, id, v[15], i[15])) return;
    v[15] = x;
    i[15] = id;
#pragma unroll
    for (int k = 15; k > 0; --k) cswap(k - 1, k);
  }
  // sort a bitonic sequence into descending order
  __device__ __forceinline__ void bitonic_merge() {
#pragma unroll
    for (int st = 8; st > 0; st >>= 1)
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if ((k & st) == 0) cswap(k, k + st);
  }
  // this <- top 16 of (this U other); both sorted descending
  __device__ __forceinline__ void merge(const float* ov, const int* oi) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const bool take = better(ov[15 - k], oi[15 - k], v[k], i[k]);
      v[k] = take ? ov[15 - k] : v[k];
      i[k] = take ? oi[15 - k] : i[k];
    }
    bitonic_merge();
  }
  // all 64 lanes of the wave end with the wave's top 16
  __device__ __forceinline__ void wave_merge() {
    // the level loop stays rolled: unrolling its six bitonic stages makes the
    // compiler's select-chain optimisations run for tens of minutes
#pragma unroll 1
    for (int s = 1; s < 64; s <<= 1) {
      float ov[16];
      int oi[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        ov[k] = __shfl_xor(v[k], s, 64);
        oi[k] = __shfl_xor(i[k], s, 64);
      }
      merge(ov, oi);
    }
  }
};

// Work-group top-16 of its lanes' lists; result valid in wave 0 (all its lanes).
__device__ __forceinline__ void block_top16(Top16& t, float* sv, int* si) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  t.wave_merge();
  if (lane < 16) {
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (k == lane) {
        sv[w * 16 + k] = t.v[k];
        si[w * 16 + k] = t.i[k];
      }
  }
  __syncthreads();
  if (w == 0) {
    t.init();
    if (lane < nw) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        t.v[k] = sv[lane * 16 + k];
        t.i[k] = si[lane * 16 + k];
      }
    }
    t.wave_merge();
  }
}

// Wave-wide top 16 of the candidates the 64 lanes hold (NV per lane, value -inf = empty).
// Exact for any input:
//   1. tau = 16th largest of the 64 lane maxima (bitonic sort across lanes).  At least 16
//      candidates are >= tau, so the top 16 are all >= tau.
//   2. Lanes compact their candidates >= tau into LDS (wave prefix sum for offsets).
//   3. Each survivor's rank under the (value desc, index asc) order is counted against all
//      survivors; rank < 16 lands in out[rank].
// When more than CAP candidates survive (heavy ties), the lanes fall back to exact
// register lists merged across the wave.  Result: out_v/out_i[0..15] in LDS.
template <int NV, int CAP>
__device__ __forceinline__ void wave_select16(const float (&v)[NV], const int (&id)[NV], float* sv, int* si,
                                              float* out_v, int* out_i) {
  const int lane = threadIdx.x & 63;
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < NV; ++j) mx = fmaxf(mx, v[j]);
  // bitonic sort of the lane maxima, descending across lanes
  float key = mx;
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const float o = __shfl_xor(key, j, 64);
      const bool up = ((lane & k) == 0);           // this lane's block sorts descending
      const bool lower = (lane & j) == 0;
      const bool keep_max = (up == lower);
      key = keep_max ? fmaxf(key, o) : fminf(key, o);
    }
  }
  const float tau = __shfl(key, 15, 64);
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < NV; ++j) cnt += (v[j] >= tau && v[j] > -INFINITY) ? 1 : 0;
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  const int total = __shfl(incl, 63, 64);
  if (total <= CAP) {
    int pos = incl - cnt;
#pragma unroll
    for (int j = 0; j < NV; ++j)
      if (v[j] >= tau && v[j] > -INFINITY) {
        sv[pos] = v[j];
        si[pos] = id[j];
        ++pos;
      }
    if (lane < 16) {
      out_v[lane] = -INFINITY;
      out_i[lane] = INT_MAX;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    for (int c = lane; c < total; c += 64) {
      const float cv = sv[c];
      const int ci = si[c];
      int rank = 0;
      for (int c2 = 0; c2 < total; ++c2) rank += better(sv[c2], si[c2], cv, ci) ? 1 : 0;
      if (rank < 16) {
        out_v[rank] = cv;
        out_i[rank] = ci;
      }
    }
  } else {
    Top16 t;
    t.init();
#pragma unroll
    for (int j = 0; j < NV; ++j) t.push(v[j], id[j]);
    t.wave_merge();
    if (lane < 16) {
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (k == lane) {
          out_v[k] = t.v[k];
          out_i[k] = t.i[k];
        }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
}

// Stage 1: top-16 of each (row, 2048-column chunk).  grid (n_chunks, rows), one wave each.
constexpr int kTopkWaveChunk = 2048;
__global__ __launch_bounds__(64) void topk_partial_kernel(const float* __restrict__ logits, int V, int ld,
                                                          float* __restrict__ pv, int32_t* __restrict__ pi) {
  constexpr int NV = kTopkWaveChunk / 64;
  __shared__ float sv[256];
  __shared__ int si[256];
  __shared__ float ov[16];
  __shared__ int oi[16];
  const int c = blockIdx.x, m = blockIdx.y, nch = gridDim.x, lane = threadIdx.x;
  const int c0 = c * kTopkWaveChunk;
  const float* row = logits + static_cast<size_t>(m) * ld;
  float v[NV];
  int id[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int col = c0 + j * 64 + lane;
    id[j] = col;
    v[j] = col < V ? row[col] : -INFINITY;
  }
  wave_select16<NV, 256>(v, id, sv, si, ov, oi);
  if (lane < 16) {
    const size_t o = (static_cast<size_t>(m) * nch + c) * 16 + lane;
    pv[o] = ov[lane];
    pi[o] = oi[lane];
  }
}

// Stage 2: merge the per-chunk lists of each row.  grid (rows), one wave; lane l takes
// lists l, l + 64, ... (at most 4 per lane), each read as four 16-byte loads.  Whole lists
// per lane keep the lane maxima high, so few candidates survive the threshold.
// Top 16 of each row of the logits (value descending, then column ascending) from the row's
// maxima over 128-column groups (tmax, written by the LM head): the 16th largest group
// maximum tau bounds the 16th largest logit from below (16 distinct columns reach it), so a
// column of a group whose maximum is below tau cannot be among the top 16.  The groups whose
// maximum is >= tau (typically 16) are scanned 16 at a time, each round's 2048 columns ranked
// together with the best 16 so far by the same comparator as the two-pass route, so the
// result is the same.  One wave per row; at most 64 * NG groups.
template <int NG>
__global__ __launch_bounds__(64) void topk_tiles_kernel(const float* __restrict__ logits, int V,
                                                        const float* __restrict__ tmax,
                                                        int32_t* __restrict__ out_ids,
                                                        float* __restrict__ out_vals) {
  __shared__ float sv[256];
  __shared__ int si[256];
  __shared__ float ov[16];
  __shared__ int oi[16];
  __shared__ int gl[64 * NG];
  const int m = blockIdx.x, lane = threadIdx.x;
  const int ng = (V + 127) / 128;
  const float* tm = tmax + static_cast<size_t>(m) * ng;
  const float* row = logits + static_cast<size_t>(m) * V;
  float v[NG];
  int id[NG];
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    const int g = lane + 64 * j;
    v[j] = g < ng ? tm[g] : -INFINITY;
    id[j] = g;
  }
  wave_select16<NG, 256>(v, id, sv, si, ov, oi);
  const float tau = ov[15];
  // the candidate groups, in increasing group order
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < NG; ++j) cnt += (lane + 64 * j < ng && v[j] >= tau) ? 1 : 0;
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  const int total = __shfl(incl, 63, 64);
  {
    int pos = incl - cnt;
#pragma unroll
    for (int j = 0; j < NG; ++j)
      if (lane + 64 * j < ng && v[j] >= tau) gl[pos++] = lane + 64 * j;
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  float bv = -INFINITY;   // lanes 0..15: the best 16 so far
  int bi = INT_MAX;
  const bool vec = (V & 3) == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0;
  for (int r0 = 0; r0 < total; r0 += 16) {
    // lane l: 32 consecutive columns of group gl[r0 + l / 4]
    float x[33];
    int xi[33];
    const int gi = r0 + (lane >> 2);
    const int col0 = (gi < total ? gl[gi] : 0) * 128 + (lane & 3) * 32;
#pragma unroll
    for (int k4 = 0; k4 < 8; ++k4) {
      const int col = col0 + 4 * k4;
      f32x4_t q = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      if (gi < total) {
        if (vec && col + 3 < V) {
          q = *reinterpret_cast<const f32x4_t*>(row + col);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) q[e] = col + e < V ? row[col + e] : -INFINITY;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[4 * k4 + e] = q[e];
        xi[4 * k4 + e] = gi < total && col + e < V ? col + e : INT_MAX;
      }
    }
    x[32] = bv;
    xi[32] = bi;
    wave_select16<33, 256>(x, xi, sv, si, ov, oi);
    bv = lane < 16 ? ov[lane] : -INFINITY;
    bi = lane < 16 ? oi[lane] : INT_MAX;
  }
  if (lane < 16) {
    out_ids[static_cast<size_t>(m) * 16 + lane] = bi;
    out_vals[static_cast<size_t>(m) * 16 + lane] = bv;
  }
}

__global__ __launch_bounds__(64) void topk_final_kernel(const float* __restrict__ pv, const int32_t* __restrict__ pi,
                                                        int n_chunks, int32_t* __restrict__ out_ids,
                                                        float* __restrict__ out_vals) {
  constexpr int LPL = 4;
  __shared__ float sv[512];
  __shared__ int si[512];
  __shared__ float ov[16];
  __shared__ int oi[16];
  const int m = blockIdx.x, lane = threadIdx.x;
  float v[16 * LPL];
  int id[16 * LPL];
#pragma unroll
  for (int q = 0; q < LPL; ++q) {
    const int c = lane + 64 * q;
    const bool ok = c < n_chunks;
    const size_t o = (static_cast<size_t>(m) * n_chunks + (ok ? c : 0)) * 16;
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      const f32x4_t fv = *reinterpret_cast<const f32x4_t*>(pv + o + 4 * k4);
      const u32x4_t iv = *reinterpret_cast<const u32x4_t*>(pi + o + 4 * k4);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[q * 16 + 4 * k4 + k] = ok ? fv[k] : -INFINITY;
        id[q * 16 + 4 * k4 + k] = ok ? static_cast<int>(iv[k]) : INT_MAX;
      }
    }
  }
  wave_select16<16 * LPL, 512>(v, id, sv, si, ov, oi);
  if (lane < 16) {
    out_ids[static_cast<size_t>(m) * 16 + lane] = oi[lane];
    out_vals[static_cast<size_t>(m) * 16 + lane] = ov[lane];
  }
}

// ------------------------------------------------------------------ greedy verification

__device__ __forceinline__ void argmax_step(float& bv, int& bi, float v, int i) {
  if (better(v, i, bv, bi)) {
    bv = v;
    bi = i;
  }
}

// Stage 1: argmax of each (target row, column chunk).  grid (n_chunks, rows), 256 threads.
// Rows are read in 16-byte vectors where the row start is 16-byte aligned, else per element.
template <typename TL>
__global__ __launch_bounds__(256) void argmax_partial_kernel(const TL* __restrict__ x, int V, int chunk,
                                                             float* __restrict__ pv, int32_t* __restrict__ pi) {
  constexpr int EPV = 16 / sizeof(TL);
  __shared__ float sv[4];
  __shared__ int si[4];
  const int c = blockIdx.x, r = blockIdx.y, nch = gridDim.x;
  const int c0 = c * chunk, c1 = min(V, c0 + chunk);
  const TL* row = x + static_cast<size_t>(r) * V;
  float bv = -INFINITY;
  int bi = INT_MAX;
  const bool vec = ((reinterpret_cast<uintptr_t>(row) & 15) == 0) && (c0 % EPV == 0);
  if (vec) {
    // four 16-byte loads per thread in flight at once (the (value, lowest id) maximum does
    // not depend on the order the elements are visited)
    constexpr int U = 4;
    const int nvec = (c1 - c0) / EPV;
    for (int q0 = threadIdx.x; q0 < nvec; q0 += 256 * U) {
      u32x4_t u[U];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int q = q0 + 256 * k;
        u[k] = q < nvec ? *reinterpret_cast<const u32x4_t*>(row + c0 + q * EPV) : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int q = q0 + 256 * k;
        if (q >= nvec) break;
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          float f;
          if constexpr (sizeof(TL) == 2) f = __uint_as_float((e & 1) ? (u[k][e >> 1] & 0xffff0000u) : (u[k][e >> 1] << 16));
          else f = __uint_as_float(u[k][e]);
          argmax_step(bv, bi, f, c0 + q * EPV + e);
        }
      }
    }
    for (int j = c0 + nvec * EPV + threadIdx.x; j < c1; j += 256) argmax_step(bv, bi, to_f<TL>(row[j]), j);
  } else {
    for (int j = c0 + threadIdx.x; j < c1; j += 256) argmax_step(bv, bi, to_f<TL>(row[j]), j);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    argmax_step(bv, bi, ov, oi);
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) {
    sv[w] = bv;
    si[w] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < 4; ++k) argmax_step(bv, bi, sv[k], si[k]);
    pv[static_cast<size_t>(r) * nch + c] = bv;
    pi[static_cast<size_t>(r) * nch + c] = bi;
  }
}

// Stage 2: per sequence, the greedy token of every row, then the accepted prefix and
// the bonus token.  grid (batch), 64 threads; n_draft <= 64.
__global__ __launch_bounds__(64) void accept_kernel(const float* __restrict__ pv, const int32_t* __restrict__ pi,
                                                    int n_chunks, const int32_t* __restrict__ draft, int n_draft,
                                                    int32_t* __restrict__ accept_len, int32_t* __restrict__ bonus) {
  __shared__ int tok[65];
  const int b = blockIdx.x, lane = threadIdx.x;
  const int R = n_draft + 1;
  for (int r = lane; r < R; r += 64) {
    const size_t o = (static_cast<size_t>(b) * R + r) * n_chunks;
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int c = 0; c < n_chunks; ++c) argmax_step(bv, bi, pv[o + c], pi[o + c]);
    tok[r] = bi;
  }
  __syncthreads();
  if (lane == 0) {
    int a = 0;
    while (a < n_draft && draft[static_cast<size_t>(b) * n_draft + a] == tok[a]) ++a;
    accept_len[b] = a;
    bonus[b] = tok[a];
  }
}

// ------------------------------------------------------------------ verification by rejection sampling
//
// p_r = softmax(target row r / t) over the vocabulary; draft i (drawn from a proposal q_i
// given sparsely by 16 ids and probabilities) is accepted when u_accept[i] * q_i(x_i) <
// p_i(x_i); at the first rejection a the bonus is drawn from max(0, p_a - q_a) (from p_a
// when every draft is accepted, or when rounding leaves that residual no mass), by
// inverting its running sum in ascending token id with u_bonus.  Exponentials are
// exp2((x - max) * k2), k2 = log2(e) / t, in fp32.

constexpr int kSoftmaxChunk = 4096;   // vocabulary columns per work-group of the stages below

// Stage 1: per (target row, column chunk) the chunk's largest logit m and
// sum exp2((x - m) * k2).  grid (n_chunks, rows), 256 threads.
template <typename TL>
__global__ __launch_bounds__(256) void softmax_partial_kernel(const TL* __restrict__ x, int V, float k2,
                                                              float* __restrict__ pm, float* __restrict__ ps) {
  __shared__ float red[4];
  const int c = blockIdx.x, r = blockIdx.y, nch = gridDim.x;
  const int c0 = c * kSoftmaxChunk, c1 = min(V, c0 + kSoftmaxChunk);
  const TL* row = x + static_cast<size_t>(r) * V;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float m = -INFINITY;
  for (int j = c0 + threadIdx.x; j < c1; j += 256) m = fmaxf(m, to_f<TL>(row[j]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if (lane == 0) red[w] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float sum = 0.f;
  for (int j = c0 + threadIdx.x; j < c1; j += 256) sum += exp2f((to_f<TL>(row[j]) - m) * k2);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
  if (lane == 0) red[w] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {
    pm[static_cast<size_t>(r) * nch + c] = m;
    ps[static_cast<size_t>(r) * nch + c] = ((red[0] + red[1]) + red[2]) + red[3];
  }
}

// What stage 2 hands to stage 3, per sequence.
struct BonusSel {
  int row;        // a: the row the bonus is drawn from
  int chunk;      // the chunk holding the draw
  int corr;       // 1: subtract the proposal of row a (a residual draw)
  float target;   // remaining mass to walk inside the chunk
  float m, inv_z; // row a's max and 1 / normaliser
};

// Stage 2: per sequence (64 threads, n_draft <= 64): row maxima and normalisers from the
// partials (chunks in ascending order), the acceptance of every draft, a, and the chunk
// of the bonus draw (residual mass per chunk; the proposal's 16 ids subtracted in order).
template <typename TL>
__global__ __launch_bounds__(64) void reject_kernel(const float* __restrict__ pm, const float* __restrict__ ps,
                                                    int nch, const TL* __restrict__ tgt, int V, float k2,
                                                    const int32_t* __restrict__ draft, int n_draft,
                                                    const int32_t* __restrict__ q_ids, long long q_stride,
                                                    const float* __restrict__ q_probs,
                                                    const float* __restrict__ u_accept,
                                                    const float* __restrict__ u_bonus,
                                                    int32_t* __restrict__ accept_len, BonusSel* __restrict__ sel) {
  __shared__ float M[65], IZ[65];
  __shared__ float R[1024];
  __shared__ int a_s;
  const int b = blockIdx.x, lane = threadIdx.x, R_rows = n_draft + 1;
  const TL* T = tgt + static_cast<size_t>(b) * R_rows * V;
  for (int r = lane; r < R_rows; r += 64) {
    const size_t o = (static_cast<size_t>(b) * R_rows + r) * nch;
    float m = -INFINITY;
    for (int c = 0; c < nch; ++c) m = fmaxf(m, pm[o + c]);
    float z = 0.f;
    for (int c = 0; c < nch; ++c) z += ps[o + c] * exp2f((pm[o + c] - m) * k2);
    M[r] = m;
    IZ[r] = 1.f / z;
  }
  __syncthreads();
  bool reject = false;
  if (lane < n_draft) {
    const int x = draft[static_cast<size_t>(b) * n_draft + lane];
    const int32_t* ids = q_ids + b * q_stride + lane * 16;
    const float* qp = q_probs + (static_cast<size_t>(b) * n_draft + lane) * 16;
    float q = 0.f;
    for (int j = 15; j >= 0; --j)
      if (ids[j] == x) q = qp[j];
    const float px = (x >= 0 && x < V) ? exp2f((to_f<TL>(T[static_cast<size_t>(lane) * V + x]) - M[lane]) * k2) * IZ[lane]
                                       : 0.f;
    reject = !(q > 0.f && u_accept[static_cast<size_t>(b) * n_draft + lane] * q < px);
  }
  const unsigned long long bal = __ballot(reject);
  const int a = bal ? __ffsll(static_cast<long long>(bal)) - 1 : n_draft;
  const float m = M[a], iz = IZ[a];
  const size_t o = (static_cast<size_t>(b) * R_rows + a) * nch;
  for (int c = lane; c < nch; c += 64) R[c] = ps[o + c] * exp2f((pm[o + c] - m) * k2) * iz;
  __syncthreads();
  if (lane == 0) {
    const int32_t* ids = q_ids + b * q_stride + a * 16;
    const float* qp = q_probs + (static_cast<size_t>(b) * n_draft + a) * 16;
    const TL* Ta = T + static_cast<size_t>(a) * V;
    float tot = 0.f;
    int corr = 0;
    if (a < n_draft) {
      for (int j = 0; j < 16; ++j) {
        const int y = ids[j];
        if (y < 0 || y >= V) continue;
        const float py = exp2f((to_f<TL>(Ta[y]) - m) * k2) * iz;
        R[y / kSoftmaxChunk] -= fminf(py, fmaxf(qp[j], 0.f));
      }
      for (int c = 0; c < nch; ++c) tot += fmaxf(R[c], 0.f);
      corr = tot > 0.f;
      if (!corr) {   // no residual mass: draw from p_a
        tot = 0.f;
        for (int c = 0; c < nch; ++c) tot += (R[c] = ps[o + c] * exp2f((pm[o + c] - m) * k2) * iz);
      }
    } else {
      for (int c = 0; c < nch; ++c) tot += R[c];
    }
    const float target = u_bonus[b] * tot;
    float run = 0.f;
    int ch = -1, last = 0;
    float rem = 0.f;
    for (int c = 0; c < nch; ++c) {
      const float rc = fmaxf(R[c], 0.f);
      if (rc > 0.f) last = c;
      if (ch < 0 && target < run + rc) {
        ch = c;
        rem = target - run;
      }
      run += rc;
    }
    if (ch < 0) {
      ch = last;
      rem = INFINITY;   // past the end through rounding: the chunk's last token of positive mass
    }
    accept_len[b] = a;
    BonusSel s;
    s.row = a;
    s.chunk = ch;
    s.corr = corr;
    s.target = rem;
    s.m = m;
    s.inv_z = iz;
    sel[b] = s;
  }
}

// Stage 3: per sequence (256 threads), the draw inside the chosen chunk: each thread walks
// 16 consecutive tokens; thread offsets by an exclusive scan in thread order.
template <typename TL>
__global__ __launch_bounds__(256) void bonus_kernel(const TL* __restrict__ tgt, int V, float k2, int n_draft,
                                                    const int32_t* __restrict__ q_ids, long long q_stride,
                                                    const float* __restrict__ q_probs,
                                                    const BonusSel* __restrict__ sel, int32_t* __restrict__ bonus) {
  constexpr int E = kSoftmaxChunk / 256;
  __shared__ int cid[16];
  __shared__ float cq[16];
  __shared__ float wsum[4];
  __shared__ int pick_s, last_s;
  const int b = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const BonusSel s = sel[b];
  if (t < 16) {
    cid[t] = s.corr ? q_ids[b * q_stride + s.row * 16 + t] : -1;
    cq[t] = s.corr ? fmaxf(q_probs[(static_cast<size_t>(b) * n_draft + s.row) * 16 + t], 0.f) : 0.f;
  }
  if (t == 0) {
    pick_s = INT_MAX;
    last_s = -1;
  }
  __syncthreads();
  const TL* row = tgt + (static_cast<size_t>(b) * (n_draft + 1) + s.row) * V;
  const int y0 = s.chunk * kSoftmaxChunk + t * E;
  float r[E];
  float sum = 0.f;
  int lastpos = -1;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int y = y0 + e;
    float v = 0.f;
    if (y < V) {
      v = exp2f((to_f<TL>(row[y]) - s.m) * k2) * s.inv_z;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (cid[j] == y) v = fmaxf(v - cq[j], 0.f);
    }
    r[e] = v;
    sum += v;
    if (v > 0.f) lastpos = y;
  }
  // inclusive scan of the thread sums in thread order; thread t owns [incl_{t-1}, incl_t),
  // both ends computed by the same operations in the two threads that share them
  float inc = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float up = __shfl_up(inc, o, 64);
    if (lane >= o) inc += up;
  }
  const float prev = __shfl_up(inc, 1, 64);
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  float base = 0.f;
  for (int k = 0; k < w; ++k) base += wsum[k];
  const float lo = lane == 0 ? base : base + prev, hi = base + inc;
  if (s.target >= lo && s.target < hi) {
    float run = lo;
    int pick = lastpos;                 // the walk can fall short of hi through rounding
#pragma unroll
    for (int e = 0; e < E; ++e) {
      run += r[e];
      if (s.target < run) {
        pick = y0 + e;
        break;
      }
    }
    atomicMin(&pick_s, pick);
  }
  if (lastpos >= 0) atomicMax(&last_s, lastpos);
  __syncthreads();
  if (t == 0) bonus[b] = pick_s != INT_MAX ? pick_s : (last_s >= 0 ? last_s : s.chunk * kSoftmaxChunk);
}

// Next cycle's state from a verified block (one thread per sequence): the anchor and the
// a accepted drafts become the next a + 1 context rows, the bonus token the next anchor.
__global__ __launch_bounds__(64) void advance_kernel(const int32_t* __restrict__ accept_len,
                                                     const int32_t* __restrict__ bonus, int B, int mask_id, int cap,
                                                     int32_t* __restrict__ ctx_len, int32_t* __restrict__ pos0,
                                                     int32_t* __restrict__ n_new, int32_t* __restrict__ block_ids) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int a = accept_len[b];
  a = a < 0 ? 0 : (a > 15 ? 15 : a);
  int L = ctx_len[b];
  L = L < 0 ? 0 : (L > cap ? cap : L);
  pos0[b] = L;
  n_new[b] = a + 1;
  ctx_len[b] = L + a + 1 > cap ? cap : L + a + 1;
  int32_t* ids = block_ids + static_cast<size_t>(b) * 16;
  ids[0] = bonus[b];
#pragma unroll
  for (int j = 1; j < 16; ++j) ids[j] = mask_id;
}

// ------------------------------------------------------------------ Path Selector

// Tokens whose 256-d embeddings are needed, per sequence: the 16 candidates of each
// drafted position p (slot 16p + j), then the anchor (slot 16P) when n_fixed = 1.
__global__ void path_tokens_kernel(const int32_t* __restrict__ cand_ids, const int32_t* __restrict__ block_ids,
                                   int n_fixed, int P, int32_t* __restrict__ tokens) {
  const int b = blockIdx.x, T = 16 * P + n_fixed;
  for (int t = threadIdx.x; t < T; t += blockDim.x) {
    const int v = t < 16 * P ? cand_ids[(static_cast<size_t>(b) * 16 + n_fixed + t / 16) * 16 + (t % 16)]
                             : block_ids[static_cast<size_t>(b) * 16];
    tokens[static_cast<size_t>(b) * T + t] = v;
  }
}

// fp32 fragment of 8 consecutive values of a T row (bf16 widened exactly)
template <typename T>
__device__ __forceinline__ f32x8_t load8_as_f32(const T* p) {
  if constexpr (std::is_same<T, float>::value) {
    return Frag<float>::load(p);
  } else {
    const u32x4_t u = *reinterpret_cast<const u32x4_t*>(p);
    f32x8_t r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r[2 * j] = __uint_as_float(u[j] << 16);
      r[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
    }
    return r;
  }
}

// Pair scores of one drafted position p of one sequence.  grid (P, B), 512 threads (8 waves:
// one 16-factor tile of U or V per wave at rank 64, so the factor loads are one round trip).
//   lam[a] = U z_l(left token a)                 (left tokens: candidates of p-1, or the anchor at p = 0)
//   rho[j] = V (gamma_p (.) z_r(candidate j of p))
//   S[p][a][j] = lam[a] . rho[j]
// lam and rho are 16 x r products on the fp32 matrix cores (K = PD); S is a plain fp32 dot
// product over r in order k = 0..r-1.  z: [B][Tn][2*PD] fp32 (left | right halves), or with
// table != nullptr the per-token table [V][2*PD] read at the tokens' ids (ids clamped to
// the vocabulary).
template <typename T>
__global__ __launch_bounds__(512) void path_scores_kernel(const float* __restrict__ z, const float* __restrict__ gamma,
                                                          const T* __restrict__ U, const T* __restrict__ Vf, int PD,
                                                          int r, int n_fixed, int P, float* __restrict__ S_out,
                                                          float* __restrict__ pair_scores,
                                                          const float* __restrict__ table,
                                                          const int32_t* __restrict__ cand_ids,
                                                          const int32_t* __restrict__ block_ids, int V) {
  extern __shared__ float sm[];
  float* lam = sm;                  // [16][r + 1]
  float* rho = sm + 16 * (r + 1);   // [16][r + 1]
  const int p = blockIdx.x, b = blockIdx.y, Tn = 16 * P + n_fixed;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;
  const bool has_left = p >= 1 || n_fixed == 1;
  float* So = S_out + ((static_cast<size_t>(b) * P + p) * 16) * 16;
  float* Po = pair_scores ? pair_scores + ((static_cast<size_t>(b) * P + p) * 16) * 16 : nullptr;
  if (!has_left) {
    for (int e = threadIdx.x; e < 256; e += blockDim.x) {
      So[e] = 0.f;
      if (Po) Po[e] = 0.f;
    }
    return;
  }
  const float* zl;
  const float* zr;
  if (table) {
    // left token of row a (p = 0: only row 0, the anchor), right token of row j
    const int32_t* cb = cand_ids + (static_cast<size_t>(b) * 16 + n_fixed) * 16;
    int tl = p >= 1 ? cb[(p - 1) * 16 + r16] : block_ids[static_cast<size_t>(b) * 16];
    int tr = cb[p * 16 + r16];
    tl = tl < 0 ? 0 : (tl >= V ? V - 1 : tl);
    tr = tr < 0 ? 0 : (tr >= V ? V - 1 : tr);
    zl = table + static_cast<size_t>(tl) * 2 * PD;
    zr = table + static_cast<size_t>(tr) * 2 * PD + PD;
  } else {
    const float* zb = z + static_cast<size_t>(b) * Tn * 2 * PD;
    // left token slot of row a (p = 0: only row 0, the anchor), right token slot of row j
    const int lslot = p >= 1 ? (p - 1) * 16 + r16 : 16 * P;
    const int rslot = p * 16 + r16;
    zl = zb + static_cast<size_t>(lslot) * 2 * PD;
    zr = zb + static_cast<size_t>(rslot) * 2 * PD + PD;
  }
  const float* gm = gamma ? gamma + (static_cast<size_t>(b) * 16 + n_fixed + p) * PD : nullptr;
  const int ntiles = (r + 15) / 16;
  const int nwaves = blockDim.x >> 6;   // 8: one 16-factor tile per wave at rank 64
  for (int job = wave; job < 2 * ntiles; job += nwaves) {
    const bool left = job < ntiles;
    const int nt = left ? job : job - ntiles;
    const int n = nt * 16 + r16;                       // output column (factor index) of this lane
    const T* wrow = (left ? U : Vf) + static_cast<size_t>(n < r ? n : 0) * PD;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    // unrolled so the loads of several k steps are in flight together (PD = 256: one batch)
#pragma unroll 8
    for (int k0 = 0; k0 < PD; k0 += 32) {
      const int k = k0 + 8 * g;
      f32x8_t a = Frag<float>::load(left ? zl + k : zr + k);
      if (!left && gm) {
        const f32x8_t gg = Frag<float>::load(gm + k);
        a *= gg;
      }
      f32x8_t w = n < r ? load8_as_f32<T>(wrow + k) : Frag<float>::zero();
      acc = Frag<float>::mma(acc, a, w);
    }
    float* dst = left ? lam : rho;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (n < r) dst[(4 * g + i) * (r + 1) + n] = acc[i];
  }
  __syncthreads();
  {
    const int a = threadIdx.x >> 4, j = threadIdx.x & 15;
    float s = 0.f;
    // (unrolled so the LDS reads of several k are in flight together; the sum stays in order)
    if (a < 16 && (p >= 1 || a == 0))
#pragma unroll 16
      for (int k = 0; k < r; ++k) s += lam[a * (r + 1) + k] * rho[j * (r + 1) + k];
    if (a < 16) {
      So[a * 16 + j] = s;
      if (Po) Po[a * 16 + j] = s;
    }
  }
}

// The pair scores and candidate logits of sequence b, staged in LDS by the 64 threads of
// the work-group: every load is issued before the first LDS store (P <= 16 float4 of S and
// 4 logits per thread), so the staging costs one memory round trip, and the walks then
// follow their chain of choices through LDS.  Ss: [P][16][16], ls: [P][16].  Ends with a
// work-group barrier.
__device__ __forceinline__ void stage_walk(const float* __restrict__ S, const float* __restrict__ lg, int P,
                                           float* Ss, float* ls) {
  const int t = threadIdx.x;   // blockDim.x == 64
  f32x4_t v[16];
  float l[4];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (i < P) v[i] = reinterpret_cast<const f32x4_t*>(S)[t + 64 * i];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (t + 64 * i < P * 16) l[i] = lg[t + 64 * i];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (i < P) reinterpret_cast<f32x4_t*>(Ss)[t + 64 * i] = v[i];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (t + 64 * i < P * 16) ls[t + 64 * i] = l[i];
  __syncthreads();
}

// The walk over the pair scores.  grid (B), 64 threads (lanes 0..15 hold one candidate each).
// Greedy: c_0 = argmax_j (l_0[j] + S[0][0][j]), c_p = argmax_j (l_p[j] + S[p][c_{p-1}][j]).
// Exact:  best_0[j] = l_0[j] + S[0][0][j]; best_p[j] = l_p[j] + max_a (best_{p-1}[a] + S[p][a][j]).
// fp32, in exactly this order; ties to the lowest index.
__global__ __launch_bounds__(64) void path_walk_kernel(const float* __restrict__ S_in,
                                                       const int32_t* __restrict__ cand_ids,
                                                       const float* __restrict__ cand_logits, int n_fixed, int P,
                                                       int mode, int32_t* __restrict__ path_idx,
                                                       int32_t* __restrict__ path_ids) {
  __shared__ float best[16];
  __shared__ int back[16][16];
  __shared__ int chosen[16];
  __shared__ __align__(16) float S[16 * 256];
  __shared__ float lg[16 * 16];
  const int b = blockIdx.x;
  stage_walk(S_in + static_cast<size_t>(b) * P * 256, cand_logits + (static_cast<size_t>(b) * 16 + n_fixed) * 16, P,
             S, lg);
  if (threadIdx.x >= 16) return;
  const int j = threadIdx.x;
  const int32_t* ci = cand_ids + (static_cast<size_t>(b) * 16 + n_fixed) * 16;
  auto argmax16 = [&](float v, int& bi) {
    float bv = v;
    bi = j;
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 16);
      const int oi = __shfl_xor(bi, o, 16);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    return bv;
  };
  if (mode == 0) {
    float sc = lg[j] + (n_fixed == 1 ? S[j] : 0.f);
    int c;
    argmax16(sc, c);
    if (j == 0) chosen[0] = c;
    for (int p = 1; p < P; ++p) {
      sc = lg[p * 16 + j] + S[(p * 16 + c) * 16 + j];
      argmax16(sc, c);
      if (j == 0) chosen[p] = c;
    }
  } else {
    float bj = lg[j] + (n_fixed == 1 ? S[j] : 0.f);
    best[j] = bj;
    for (int p = 1; p < P; ++p) {
      __builtin_amdgcn_wave_barrier();
      float bv = -INFINITY;
      int ba = 0;
      for (int a = 0; a < 16; ++a) {
        const float v = best[a] + S[(p * 16 + a) * 16 + j];
        if (v > bv) {
          bv = v;
          ba = a;
        }
      }
      back[p][j] = ba;
      bj = lg[p * 16 + j] + bv;
      __builtin_amdgcn_wave_barrier();
      best[j] = bj;
    }
    __builtin_amdgcn_wave_barrier();
    int c;
    argmax16(bj, c);
    if (j == 0) {
      for (int p = P - 1; p >= 0; --p) {
        chosen[p] = c;
        if (p > 0) c = back[p][c];
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  for (int p = j; p < P; p += 16) {
    const int c = chosen[p];
    path_idx[static_cast<size_t>(b) * P + p] = c;
    path_ids[static_cast<size_t>(b) * P + p] = ci[p * 16 + c];
  }
}

// The sampled walk: q_p[j] = softmax_j of the greedy walk's score of candidate j at
// temperature t (scores scaled by k2 = log2(e)/t; max and sum by a 16-lane butterfly),
// and c_p = the first j whose running sum of q_p (candidate order) exceeds
// uniforms[b][p] times the total (the last j with q_p > 0 if none does).  grid (B), 64
// threads (lanes 0..15 hold one candidate each).
__global__ __launch_bounds__(64) void path_sample_kernel(const float* __restrict__ S_in,
                                                         const int32_t* __restrict__ cand_ids,
                                                         const float* __restrict__ cand_logits, int n_fixed, int P,
                                                         float k2,
                                                         const float* __restrict__ uniforms,
                                                         int32_t* __restrict__ path_idx,
                                                         int32_t* __restrict__ path_ids,
                                                         float* __restrict__ path_q) {
  __shared__ __align__(16) float S[16 * 256];
  __shared__ float lg[16 * 16];
  const int b = blockIdx.x;
  stage_walk(S_in + static_cast<size_t>(b) * P * 256, cand_logits + (static_cast<size_t>(b) * 16 + n_fixed) * 16, P,
             S, lg);
  if (threadIdx.x >= 16) return;
  const int j = threadIdx.x;
  const int32_t* ci = cand_ids + (static_cast<size_t>(b) * 16 + n_fixed) * 16;
  int c = 0;
  for (int p = 0; p < P; ++p) {
    const float sc = p == 0 ? lg[j] + (n_fixed == 1 ? S[j] : 0.f) : lg[p * 16 + j] + S[(p * 16 + c) * 16 + j];
    float mx = sc;
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 16));
    const float e = exp2f((sc - mx) * k2);
    float z = e;
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) z += __shfl_xor(z, o, 16);
    const float q = e / z;
    path_q[(static_cast<size_t>(b) * P + p) * 16 + j] = q;
    float tot = 0.f;
    for (int i = 0; i < 16; ++i) tot += __shfl(q, i, 16);
    const float target = uniforms[static_cast<size_t>(b) * P + p] * tot;
    float run = 0.f;
    int pick = -1, last = 0;
    for (int i = 0; i < 16; ++i) {
      const float qi = __shfl(q, i, 16);
      run += qi;
      if (pick < 0 && target < run) pick = i;
      if (qi > 0.f) last = i;
    }
    c = pick >= 0 ? pick : last;
    if (j == 0) {
      path_idx[static_cast<size_t>(b) * P + p] = c;
      path_ids[static_cast<size_t>(b) * P + p] = ci[p * 16 + c];
    }
  }
}

}  // namespace dflash
