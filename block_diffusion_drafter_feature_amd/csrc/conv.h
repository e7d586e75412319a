// The DFlash 2 dynamic short convolution, one fused kernel per conv site ("DFlash 2:
// optimización ...", "Arquitectura del Sistema", item 2: two taps along the block, depthwise,
// coefficients that follow the current row, one correction per 16 channels, before and after
// every attention and FFN sublayer).
//
// For block row t of a sequence (rows 16b .. 16b+15, u_{-1} = 0):
//   delta_t = bf16(u_t) W_gen^T                          (2 * d/16 corrections)
//   y_t[c]  = u_t[c] + (w0[c] + delta_t[c/16]) u_t[c] + (w1[c] + delta_t[d/16 + c/16]) u_{t-1}[c]
//
// One work-group per (tile of 16 channel groups = 256 channels, sequence).  Its eight waves
// split K (the row width d) by 32-wide k-steps and compute the 16 x 32 block of corrections
// the tile needs -- the 16 "current row" generator rows of its groups and their 16 "previous
// row" partners -- on the matrix cores, reduce them through LDS in a fixed order, and then
// apply both taps to the tile's 256 channels of the 16 rows.  Nothing is written between the
// correction and its use, so one launch covers a site.
//
// PRE (the conv on a sublayer's normed input): u = RMSNorm(x; gain) is formed inside the
// kernel -- each work-group reads its 16 residual rows once for the row scales and again as
// the matrix-core operand -- and y goes out rounded to the storage type (the next GEMM's A
// operand).  With emb/ids the residual rows are first gathered from the embedding (the
// block's first layer); the work-group of tile 0 stores them to x.
// POST (the conv on a sublayer's output): u is the sublayer GEMM's fp32 output and y is added
// to the residual stream x.
#pragma once

#include "common.h"

namespace dflash {

constexpr int kConvWaves = 8;       // waves per work-group (K split)
// k-steps per stage (all of a stage's loads in flight together): 8 for bf16, 4 for fp32 operands
template <typename T>
constexpr int conv_stage() { return sizeof(T) == 2 ? 8 : 4; }

// 8 consecutive elements of T (16- or 32-byte aligned) as floats
template <typename T>
__device__ __forceinline__ void load8f(const T* p, float (&v)[8]) {
  if constexpr (sizeof(T) == 4) {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[4 + e] = b[e];
    }
  } else {
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[e] << 16);
      v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  }
}

// Per-wave LDS staging of the corrections' operands (bf16 weights, rows not gathered): slot I
// of wave w holds one 64-k slab -- the 16 fp32 rows (4 KB, chunk c of row r at position
// c ^ (r & 15)) and the tile's 32 generator rows (4 KB, chunk c of row r at c ^ ((r >> 1) & 7)),
// both filled by direct loads (dma16) that the wave waits for itself, and (PRE) the slab's 64
// RMSNorm gains (128 B, loaded twice by a 4-byte-per-lane direct load).  Fragment-shaped loads straight into
// registers (16 rows x 64 B per instruction) stream these operands at well under half the
// rate (~33 against ~74 GB/s per work-group).
constexpr int kConvSlabBytes = 8192 + 256;

// 4 bytes per lane from global address g into LDS at (wave-uniform) byte address lds + 4 * lane
// (untracked by the compiler, as dma16)
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}
template <int I>
__device__ __forceinline__ char* conv_ring() {
  __shared__ __attribute__((aligned(16))) char s[kConvWaves * kConvSlabBytes];
  return s;
}



template <typename T, bool PRE>
__global__ __launch_bounds__(64 * kConvWaves) void conv_site_kernel(
    const float* __restrict__ src,      // PRE: residual x (unless gathering); POST: sublayer output
    const T* __restrict__ emb, const int32_t* __restrict__ ids,   // PRE, first layer: gather x = E[ids]
    const float* __restrict__ ss_in, int n_ss,   // PRE: partial sums of squares of x rows [M][n_ss]
    const T* __restrict__ gain, float eps,       // PRE: RMSNorm gain and epsilon
    const T* __restrict__ gen, const T* __restrict__ w0, const T* __restrict__ w1, int d,
    float* __restrict__ x,              // PRE: written with the gathered rows (tile 0); POST: x += y
    float* __restrict__ ss_out,         // POST: partial sums of squares of the new x rows [M][gridDim.x]
    T* __restrict__ out) {              // PRE: y rounded to T
  typedef Frag<T> F;
  typedef typename F::type frag_t;
  constexpr int NW = kConvWaves, U = conv_stage<T>();
  __shared__ float red[NW][2][256];
  __shared__ float dlt[2][16][17];      // [tap][row][group in tile]
  __shared__ float inv_s[16];
  __shared__ float ssp[2][4][8];        // POST: [row half][wave][row] partial sums of squares

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  // Work-groups are dealt to the 8 XCDs round-robin in dispatch order (x fastest).  When the
  // grid allows, consecutive work-groups of one XCD take a block of 4 sequences x 8 channel
  // tiles, so that XCD's L2 holds those sequences' rows and those tiles' generator rows
  // (otherwise every XCD would fetch every sequence's rows).  A bijection of the grid.
  int tile = blockIdx.x, seq = blockIdx.y;
  {
    const int nt = gridDim.x, ns = gridDim.y, n = nt * ns;
    if (nt % 8 == 0 && ns % 4 == 0) {
      const int L = blockIdx.y * nt + blockIdx.x;
      const int W = (L % 8) * (n / 8) + L / 8;
      const int r = W % (4 * nt);
      seq = (W / (4 * nt)) * 4 + r % 4;
      tile = r / 4;
    }
  }
  const int ng = d >> 4, g0 = tile * 16;
  const size_t m0 = static_cast<size_t>(seq) * 16;
  const bool gather = PRE && emb != nullptr;

  // row r of this block as fp32: the residual / the sublayer output (unused when gathering)
  auto row_ptr_f = [&](int r) { return src + (m0 + r) * d; };
  const T* erow = gather ? emb + static_cast<size_t>(ids[m0 + r16]) * d : nullptr;

  // ---- PRE: row scales 1 / sqrt(mean(x^2) + eps)
  if constexpr (PRE) {
    if (ss_in) {
      // the producer of x left per-row partial sums (fixed order here)
      if (tid < 16) {
        float ss = 0.f;
        for (int i = 0; i < n_ss; ++i) ss += ss_in[(m0 + tid) * n_ss + i];
        inv_s[tid] = 1.f / sqrtf(ss / d + eps);
      }
    } else {
      // from the rows themselves, 32 threads per row, eight 16-byte loads in flight per thread
      const int r = tid >> 5, q = tid & 31;
      float ss = 0.f;
      if (r < 16) {
        const T* er = gather ? emb + static_cast<size_t>(ids[m0 + r]) * d : nullptr;
        const float* xr = row_ptr_f(r);
        for (int c0 = 4 * q; c0 < d; c0 += 128 * 8) {
          f32x4_t v[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int c = c0 + 128 * i;
            if (c < d) {
              if (gather) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[i][e] = to_f<T>(er[c + e]);
              } else {
                v[i] = *reinterpret_cast<const f32x4_t*>(xr + c);
              }
            } else {
              v[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int c = c0 + 128 * i;
            if (gather && tile == 0 && c < d) *reinterpret_cast<f32x4_t*>(x + (m0 + r) * d + c) = v[i];
            ss += v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3];
          }
        }
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 32);
        if (q == 0) inv_s[r] = 1.f / sqrtf(ss / d + eps);
      }
    }
  }

  // ---- corrections of the tile's groups: [16 rows] x [16 current-row taps | 16 previous-row taps]
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(gen, static_cast<uint32_t>(static_cast<size_t>(2 * ng) * d * sizeof(T)));
  const uint32_t oa = static_cast<uint32_t>((static_cast<size_t>(g0 + r16) * d + g * 8) * sizeof(T));
  const uint32_t ob = static_cast<uint32_t>((static_cast<size_t>(ng + g0 + r16) * d + g * 8) * sizeof(T));
  const uint32_t past = static_cast<uint32_t>(static_cast<size_t>(2 * ng) * d * sizeof(T));   // reads zero
  const float* arow = row_ptr_f(r16);

  f32x4_t acc_a{0.f, 0.f, 0.f, 0.f}, acc_b{0.f, 0.f, 0.f, 0.f};
  const int nks = d / 32;
  bool staged = false;
  if constexpr (sizeof(T) == 2) staged = !gather;
  if (staged) {
    if constexpr (sizeof(T) == 2) {
      // wave w takes the 64-k slabs w, w + NW, ...; two slots per wave, the next slab's loads
      // in flight while one is consumed (each wave reads only its own slots: no barrier)
      constexpr int LPS = PRE ? 9 : 8;   // 4 row loads + 4 generator loads (+ the gains) per slab
      const int nsl = d / 64, ntw = wave < nsl ? (nsl - 1 - wave) / NW + 1 : 0;
      float inv = 1.f;         // (PRE) this lane's row scale

      char* const sl0 = conv_ring<0>() + wave * kConvSlabBytes;
      char* const sl1 = conv_ring<1>() + wave * kConvSlabBytes;
      auto issue = [&](int v, int t) {
        const int k0 = 64 * (wave + NW * (t < ntw ? t : ntw - 1));
        const uint32_t b = lds_addr(v ? sl1 : sl0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = 4 * j + (lane >> 4), c = (lane & 15) ^ row;
          dma16(row_ptr_f(row) + k0 + 4 * c, b + j * 1024);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {   // rows past the 2 ng generator rows (unused groups) read row 0
          const int row = 8 * j + (lane >> 3), c = (lane & 7) ^ ((row >> 1) & 7);
          const int grow = row < 16 ? g0 + row : ng + g0 + row - 16;
          dma16(gen + static_cast<size_t>(grow < 2 * ng ? grow : 0) * d + k0 + 8 * c, b + 4096 + j * 1024);
        }
        if constexpr (PRE) dma4(gain + k0 + 2 * (lane & 31), b + 8192);


      };
      auto step = [&](int v, int t) {
        __builtin_amdgcn_s_waitcnt((LPS & 15) | ((LPS >> 4) << 14) | (7 << 4));   // slab t is in
        asm volatile("" ::: "memory");
        const char* b = v ? sl1 : sl0;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int c0 = 8 * q + 2 * g;
          const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(b + r16 * 256 + ((c0 ^ r16) << 4));
          const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(b + r16 * 256 + (((c0 + 1) ^ r16) << 4));
          float av[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          if constexpr (PRE) {
            const u32x4_t gv4 = *reinterpret_cast<const u32x4_t*>(b + 8192 + (32 * q + 8 * g) * sizeof(T));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t gw = gv4[e];
              av[2 * e] = av[2 * e] * inv * __uint_as_float(gw << 16);
              av[2 * e + 1] = av[2 * e + 1] * inv * __uint_as_float(gw & 0xffff0000u);
            }
          }
          const frag_t a = F::from_floats(av);
          const int pw = ((4 * q + g) ^ ((r16 >> 1) & 7)) << 4;
          const frag_t wa = *reinterpret_cast<const frag_t*>(b + 4096 + r16 * 128 + pw);
          const frag_t wb = *reinterpret_cast<const frag_t*>(b + 4096 + (16 + r16) * 128 + pw);
          acc_a = F::mma(acc_a, a, wa);
          acc_b = F::mma(acc_b, a, wb);
        }
        // this slot's reads must have completed before its next slab's direct loads can land
        __builtin_amdgcn_s_waitcnt(0xc07f);
        issue(v, t + 2);
      };
      if (ntw > 0) {
        issue(0, 0);
        issue(1, 1);
      }
      if constexpr (PRE) {   // the row scales are in LDS (a barrier without a memory fence)
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_s_barrier();
        inv = inv_s[r16];
      }
      if (ntw == 8) {   // d = 4096: straight-line code keeps the compiler's wait counting exact
#pragma unroll
        for (int t = 0; t < 8; t += 2) {
          step(0, t);
          step(1, t + 1);
        }
      } else {
        int t = 0;
        for (; t + 2 <= ntw; t += 2) {
          step(0, t);
          step(1, t + 1);
        }
        if (t < ntw) step(0, t);
      }
      __builtin_amdgcn_s_waitcnt(0);   // the re-reads past the wave's last slab
      asm volatile("" ::: "memory");
    }
  } else {
    // wave w takes k-steps w, w + NW, w + 2 NW, ...: U of them per stage, all of a stage's
    // loads issued together (A as raw fp32 rows, scaled and rounded once the row scales are in)
    for (int s0 = wave; s0 < nks; s0 += NW * U) {
      float av[U][8], gv[U][8];
      frag_t wa[U], wb[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ks = s0 + u * NW;
        const bool ok = ks < nks;
        const int k = ok ? 32 * ks + 8 * g : 0;
        const uint32_t koff = static_cast<uint32_t>(ks * 32 * sizeof(T));
        if (gather) load8f<T>(erow + k, av[u]);
        else load8f<float>(arow + k, av[u]);
        if constexpr (PRE) load8f<T>(gain + k, gv[u]);
        wa[u] = F::load_buf(rg, ok ? oa + koff : past, 0);
        wb[u] = F::load_buf(rg, ok ? ob + koff : past, 0);
      }
      if (PRE && s0 == wave) __syncthreads();   // the row scales are in LDS
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool ok = s0 + u * NW < nks;
        if constexpr (PRE) {
          const float inv = inv_s[r16];
#pragma unroll
          for (int e = 0; e < 8; ++e) av[u][e] = av[u][e] * inv * gv[u][e];
        }
        const frag_t a = ok ? F::from_floats(av[u]) : F::zero();
        acc_a = F::mma(acc_a, a, wa[u]);
        acc_b = F::mma(acc_b, a, wb[u]);
      }
    }
    if (PRE && wave >= nks) __syncthreads();    // waves without k-steps meet the row-scale barrier too
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    red[wave][0][lane * 4 + i] = acc_a[i];
    red[wave][1][lane * 4 + i] = acc_b[i];
  }
  __syncthreads();
  {
    // fixed-order sum over the waves; element e = 4 lane + i holds row 4 (lane / 16) + i,
    // group lane % 16 of tap e / 256
    const int tap = tid >> 8, e = tid & 255;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += red[w][tap][e];
    const int l = e >> 2, i = e & 3;
    dlt[tap][4 * (l >> 4) + i][l & 15] = s;
  }
  __syncthreads();

  // ---- apply both taps: thread t owns channel 16 g0 + (t % 256) over rows 8 (t / 256) .. +7
  const int c = 16 * g0 + (tid & 255), jg = (tid & 255) >> 4;
  const bool live = g0 + jg < ng;
  const int rb = (tid >> 8) * 8;
  float uv[9], xv[8];
#pragma unroll
  for (int r = 0; r < 9; ++r) {        // uv[0] = row rb - 1 (zero above row 0)
    const int row = rb - 1 + r;
    float v = 0.f;
    if (live && row >= 0) {
      v = gather ? to_f<T>(emb[static_cast<size_t>(ids[m0 + row]) * d + c]) : row_ptr_f(row)[c];
      if constexpr (PRE) v *= inv_s[row];
    }
    uv[r] = v;
  }
  if constexpr (!PRE) {
#pragma unroll
    for (int r = 0; r < 8; ++r) xv[r] = live ? x[(m0 + rb + r) * d + c] : 0.f;
  }
  const float a0 = live ? to_f<T>(w0[c]) : 0.f, b0 = live ? to_f<T>(w1[c]) : 0.f;
  const float gc = PRE && live ? to_f<T>(gain[c]) : 1.f;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const float ur = uv[r + 1] * gc, prev = uv[r] * gc;
    const float a = a0 + dlt[0][rb + r][jg], bb = b0 + dlt[1][rb + r][jg];
    const float y = ur + a * ur + bb * prev;
    if constexpr (PRE) {
      if (live) out[(m0 + rb + r) * d + c] = from_f<T>(y);
    } else {
      xv[r] += y;
      if (live) x[(m0 + rb + r) * d + c] = xv[r];
    }
  }
  if constexpr (!PRE) {
    // partial sums of squares of the new rows over this tile's channels: per wave (fixed tree),
    // then the four waves of a row half in order
    if (ss_out) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float s = wave_sum(live ? xv[r] * xv[r] : 0.f);
        if (lane == 0) ssp[tid >> 8][wave & 3][r] = s;
      }
      __syncthreads();
      if (tid < 16) {
        const int h = tid >> 3, r = tid & 7;
        const float s = ((ssp[h][0][r] + ssp[h][1][r]) + ssp[h][2][r]) + ssp[h][3][r];
        ss_out[(m0 + tid) * gridDim.x + tile] = s;
      }
    }
  }
}

}  // namespace dflash
