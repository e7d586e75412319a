// GEMMs of the drafting step on the gfx950 matrix cores:  C[m, n] = sum_k A[m, k] W[n, k].
//
// A is an activation matrix (row-major, optional row gather, given either in the
// storage type T or in fp32 and rounded to T as it is loaded).  W rows are looked
// up through the epilogue functor, which maps a "virtual 16-column tile" and a
// column inside it to a weight row.  That indirection lets one launch cover
// several weight matrices (Q|K|V, the K/V projections of every layer) and lets a
// tile hold columns that belong together (a RoPE pair d, d+hd/2; a gate/up pair)
// so the epilogue can combine them without another pass.
//
// Two kernels:
//  * gemm_skinny : M <= 64 (the drafted block of 1..4 sequences).  Weight
//    streaming: each work-group owns NT virtual tiles over the whole K; its NW
//    waves split K, stream their slice of W straight from HBM into registers
//    (16 B per lane per fragment, two register stages in flight) and reduce
//    through LDS in a fixed order.
//  * gemm_tiled  : M > 64.  128x128 output tile per work-group, A and W tiles
//    staged through LDS (register prefetch of the next K slab while the matrix
//    cores work on the current one), 2x2 waves of 64x64.
// Both are deterministic (no atomics).
#pragma once

#include "common.h"
#include <type_traits>

namespace dflash {

template <typename T, typename AS>
__device__ __forceinline__ typename Frag<T>::type load_a(const AS* p) {
  if constexpr (std::is_same<AS, T>::value) return Frag<T>::load(p);
  else return Frag<T>::load_f32(p);
}

// ---------------------------------------------------------------------------------
// skinny GEMM
// ---------------------------------------------------------------------------------

// NT virtual tiles per work-group (and per wave), NW waves splitting K, U k-steps per
// register stage.  Two register stages alternate: the loads of stage i+1 are in flight
// while the matrix cores consume stage i.
template <typename T, typename AS, int MT, int NT, int NW, int U, class Epi>
__global__ __launch_bounds__(64 * NW) void gemm_skinny_kernel(const AS* __restrict__ A, int lda,
                                                              const int32_t* __restrict__ arows, int M, int K,
                                                              Epi epi) {
  typedef Frag<T> F;
  typedef typename F::type frag_t;
  constexpr int ROWS = 16 * MT;
  constexpr int TW = 16 * NT;
  __shared__ float red[NW][MT * NT * 256];
  __shared__ float tile[ROWS][TW + 1];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int vt0 = blockIdx.x * NT;

  // W through one buffer descriptor per tile (rows past the matrix read as zero); A rows
  // past M are clamped to row 0 (their results are never stored).  No per-load predicates.
  const int kw = K / NW;
  const int k0 = wave * kw;
  __amdgpu_buffer_rsrc_t rw[NT];
  uint32_t vw[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const T* base;
    uint32_t bytes;
    epi.wseg(vt0 + nt, base, bytes);
    rw[nt] = make_rsrc(base, bytes);
    const T* p = epi.wrow(vt0 + nt, r16);
    vw[nt] = p ? static_cast<uint32_t>((p - base + g * 8 + k0) * sizeof(T)) : bytes;
  }
  const AS* ap[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + r16;
    const int ar = m < M ? (arows ? arows[m] : m) : (arows ? arows[0] : 0);
    ap[mt] = A + static_cast<size_t>(ar) * lda + g * 8 + k0;
  }

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  constexpr int STEP = 32 * U;   // K elements per register stage
  auto load = [&](frag_t (&w)[U][NT], frag_t (&a)[U][MT], int kb) {
    const int soff = kb * static_cast<int>(sizeof(T));
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) w[u][nt] = F::load_buf(rw[nt], vw[nt] + 32 * u * sizeof(T), soff);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) a[u][mt] = load_a<T, AS>(ap[mt] + kb + 32 * u);
    }
  };
  auto mma = [&](frag_t (&w)[U][NT], frag_t (&a)[U][MT]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = F::mma(acc[mt][nt], a[u][mt], w[u][nt]);
  };

  // wave-uniform K loop over this wave's slice [k0, k0 + kw), kw a multiple of STEP.  The
  // next stage's loads are issued before the current stage's matrix ops; the prefetched
  // stage is then carried into the next iteration (one loop-carried stage, updated by copy).
  const int nst = kw / STEP;
  frag_t wc[U][NT], ac[U][MT];
  load(wc, ac, 0);
  for (int st = 1; st < nst; ++st) {
    frag_t wn[U][NT], an[U][MT];
    load(wn, an, st * STEP);
    mma(wc, ac);
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) wc[u][nt] = wn[u][nt];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) ac[u][mt] = an[u][mt];
    }
  }
  mma(wc, ac);

  // fixed-order reduction of the NW partial tiles
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][((mt * NT + nt) * 64 + lane) * 4 + i] = acc[mt][nt][i];
  __syncthreads();
  for (int e = threadIdx.x; e < MT * NT * 256; e += 64 * NW) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += red[w][e];
    const int i = e & 3, l = (e >> 2) & 63, t = e >> 8;
    const int mt = t / NT, nt = t % NT;
    tile[mt * 16 + 4 * (l >> 4) + i][nt * 16 + (l & 15)] = s;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < ROWS * TW; e += 64 * NW) {
    const int m = e / TW, c = e % TW;
    if (m >= M) continue;
    const int pc = (((c >> 4) ^ Epi::PX) << 4) | ((c & 15) ^ Epi::PC);
    epi.apply(vt0 + (c >> 4), m, c & 15, tile[m][c], tile[m][pc]);
  }
}

// ---------------------------------------------------------------------------------
// tiled GEMM (M > 64)
// ---------------------------------------------------------------------------------

template <typename T> struct TiledCfg;
template <> struct TiledCfg<bf16_t> { static constexpr int BK = 64; };
template <> struct TiledCfg<float> { static constexpr int BK = 32; };

// With partial != nullptr (split-K), work-group z covers K range [z*kslice, (z+1)*kslice)
// and stores its raw fp32 tile to partial[z][m][ldp] instead of running the epilogue.
template <typename T, typename AS, class Epi>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(const AS* __restrict__ A, int lda,
                                                         const int32_t* __restrict__ arows, int M, int K,
                                                         Epi epi, int kslice, float* __restrict__ partial,
                                                         int ldp) {
  typedef Frag<T> F;
  typedef typename F::type frag_t;
  constexpr int BM = 128, BN = 128, BK = TiledCfg<T>::BK;
  constexpr int EPB = 16 / sizeof(T);           // elements per 16-byte chunk
  constexpr int CPR = BK / EPB;                 // chunks per tile row (8)
  constexpr int LD = BK + EPB;                  // padded LDS row (elements)
  constexpr int CH = BM * CPR / 256;            // chunks per thread per operand (4)
  constexpr int SMEM_AB = 2 * BM * LD * sizeof(T);
  constexpr int SMEM_EP = 64 * (BN + 1) * sizeof(float);
  constexpr int SMEM = SMEM_AB > SMEM_EP ? SMEM_AB : SMEM_EP;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  T* As = reinterpret_cast<T*>(smem);
  T* Bs = As + BM * LD;
  float* Ct = reinterpret_cast<float*>(smem);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM;
  const int vt0 = blockIdx.x * (BN / 16);

  // global->register staging: chunk q of this thread covers row (tid*CH+q)/CPR, chunk (tid*CH+q)%CPR
  const AS* agp[CH];
  const T* bgp[CH];
  bool aok[CH];
#pragma unroll
  for (int q = 0; q < CH; ++q) {
    const int idx = tid * CH + q, r = idx / CPR, ck = idx % CPR;
    const int m = m0 + r;
    aok[q] = m < M;
    const int ar = aok[q] ? (arows ? arows[m] : m) : 0;
    agp[q] = A + static_cast<size_t>(ar) * lda + ck * EPB;
    const T* wr = epi.wrow(vt0 + r / 16, r % 16);
    bgp[q] = wr ? wr + ck * EPB : nullptr;
  }
  u32x4_t ra[CH], rb[CH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      if (aok[q]) {
        if constexpr (std::is_same<AS, T>::value) {
          ra[q] = *reinterpret_cast<const u32x4_t*>(agp[q] + k0);
        } else {  // fp32 source rounded to bf16: 8 values -> one 16 B chunk
          ra[q] = __builtin_bit_cast(u32x4_t, Frag<T>::load_f32(reinterpret_cast<const float*>(agp[q]) + k0));
        }
      } else {
        ra[q] = u32x4_t{0u, 0u, 0u, 0u};
      }
      rb[q] = bgp[q] ? *reinterpret_cast<const u32x4_t*>(bgp[q] + k0) : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      const int idx = tid * CH + q, r = idx / CPR, ck = idx % CPR;
      *reinterpret_cast<u32x4_t*>(As + r * LD + ck * EPB) = ra[q];
      *reinterpret_cast<u32x4_t*>(Bs + r * LD + ck * EPB) = rb[q];
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int kofs = blockIdx.z * kslice;
  const int KT = (partial ? kslice : K) / BK;
  gload(kofs);
  sstore();
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) gload(kofs + (kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      frag_t af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = F::load(As + (wm * 64 + i * 16 + r16) * LD + ks * 32 + g * 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) bfr[j] = F::load(Bs + (wn * 64 + j * 16 + r16) * LD + ks * 32 + g * 8);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = F::mma(acc[i][j], af[i], bfr[j]);
    }
    __syncthreads();
    if (kt + 1 < KT) {
      sstore();
      __syncthreads();
    }
  }

  if (partial) {
    float* pz = partial + static_cast<size_t>(blockIdx.z) * M * ldp;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + wm * 64 + i * 16 + 4 * g + e;
          if (m < M) pz[static_cast<size_t>(m) * ldp + vt0 * 16 + wn * 64 + j * 16 + r16] = acc[i][j][e];
        }
    return;
  }
  // epilogue, one 64-row half at a time through LDS
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wm == half) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            Ct[(i * 16 + 4 * g + e) * (BN + 1) + wn * 64 + j * 16 + r16] = acc[i][j][e];
    }
    __syncthreads();
    for (int e = tid; e < 64 * BN; e += 256) {
      const int r = e / BN, c = e % BN;
      const int m = m0 + half * 64 + r;
      if (m < M) {
        const int pc = (((c >> 4) ^ Epi::PX) << 4) | ((c & 15) ^ Epi::PC);
        epi.apply(vt0 + (c >> 4), m, c & 15, Ct[r * (BN + 1) + c], Ct[r * (BN + 1) + pc]);
      }
    }
    __syncthreads();
  }
}

// Split-K reduction: sum the partial tiles in z order, then the epilogue.  One thread per
// (row, virtual column).
template <class Epi>
__global__ __launch_bounds__(256) void gemm_splitk_epilogue_kernel(const float* __restrict__ partial, int M,
                                                                   int ldp, int ks, int n_vtiles, Epi epi) {
  const size_t e = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= static_cast<size_t>(M) * ldp) return;
  const int m = static_cast<int>(e / ldp), col = static_cast<int>(e % ldp);
  const int vt = col >> 4, c = col & 15;
  if (vt >= n_vtiles) return;
  const int pcol = ((vt ^ Epi::PX) << 4) | (c ^ Epi::PC);
  float v = 0.f, pv = 0.f;
  for (int z = 0; z < ks; ++z) {
    const float* pz = partial + static_cast<size_t>(z) * M * ldp + static_cast<size_t>(m) * ldp;
    v += pz[col];
    pv += pz[pcol];
  }
  epi.apply(vt, m, c, v, pv);
}

// ---------------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------------

// Split-K factor of the tiled GEMM: split K only when the output tiles alone cannot
// fill the 256 compute units; keep >= 2 K slabs per split.
template <typename T>
inline int splitk_plan(int M, int K, int n_vtiles) {
  if (M <= 64) return 1;
  const int BK = TiledCfg<T>::BK;
  const int tiles = ((n_vtiles + 7) / 8) * ((M + 127) / 128);
  if (tiles >= 192) return 1;
  int ks = (256 + tiles - 1) / tiles;
  ks = ks > 8 ? 8 : ks;
  const int slabs = K / BK;
  while (ks > 1 && (slabs % ks || slabs / ks < 2)) --ks;
  return ks;
}

template <typename T>
inline size_t splitk_scratch_bytes(int M, int K, int n_vtiles) {
  const int ks = splitk_plan<T>(M, K, n_vtiles);
  return ks > 1 ? static_cast<size_t>(ks) * M * (((n_vtiles + 7) / 8) * 128) * sizeof(float) : 0;
}

// Skinny launch configuration (measured on MI355X with cold caches, M = 16, bf16): two
// tiles per wave (a gate/up pair for SwiGLU) and K split over 4 waves when there are at
// least 192 such work-groups and K <= 8192; one tile per wave and K split over 8 waves
// otherwise; 8 k-steps per register stage at M = 16.  K must be
// a multiple of NW * 32 * U; smaller splits are used when it is not.
template <typename T, typename AS, int MT, int NT, int NW, int U, class Epi>
static bool try_skinny(const AS* A, int lda, const int32_t* arows, int M, int K, int n_vtiles, const Epi& epi,
                       hipStream_t s) {
  if (K % (NW * 32 * U) || n_vtiles % NT) return false;
  gemm_skinny_kernel<T, AS, MT, NT, NW, U, Epi><<<n_vtiles / NT, 64 * NW, 0, s>>>(A, lda, arows, M, K, epi);
  return true;
}

template <typename T, typename AS, int MT, class Epi>
static hipError_t launch_skinny(const AS* A, int lda, const int32_t* arows, int M, int K, int n_vtiles,
                                const Epi& epi, hipStream_t s) {
  constexpr int U = MT >= 4 ? 2 : (MT == 2 ? 4 : 8);
  const bool wide = n_vtiles / 2 >= 192 && K <= 8192;
  bool ok = false;
  if (wide || Epi::PX) ok = try_skinny<T, AS, MT, 2, 4, U>(A, lda, arows, M, K, n_vtiles, epi, s);
  if (!ok && !Epi::PX) ok = try_skinny<T, AS, MT, 1, 8, U>(A, lda, arows, M, K, n_vtiles, epi, s);
  if (!ok && !Epi::PX) ok = try_skinny<T, AS, MT, 1, 8, 2>(A, lda, arows, M, K, n_vtiles, epi, s);
  if (!ok) ok = try_skinny<T, AS, MT, (Epi::PX ? 2 : 1), 4, 1>(A, lda, arows, M, K, n_vtiles, epi, s);
  if (!ok) ok = try_skinny<T, AS, MT, (Epi::PX ? 2 : 1), 2, 1>(A, lda, arows, M, K, n_vtiles, epi, s);
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

// n_vtiles: number of virtual 16-column tiles (multiple of 2 when Epi::PX == 1).
// K: multiple of 64.  scratch: split-K partials (>= splitk_scratch_bytes, or nullptr: no split).
template <typename T, typename AS, class Epi>
static hipError_t run_gemm(const AS* A, int lda, const int32_t* arows, int M, int K, int n_vtiles, const Epi& epi,
                           hipStream_t s, float* scratch = nullptr, size_t scratch_bytes = 0) {
  if (M <= 0 || n_vtiles <= 0) return hipSuccess;
  if (M <= 16) return launch_skinny<T, AS, 1>(A, lda, arows, M, K, n_vtiles, epi, s);
  if (M <= 32) return launch_skinny<T, AS, 2>(A, lda, arows, M, K, n_vtiles, epi, s);
  if (M <= 64) return launch_skinny<T, AS, 4>(A, lda, arows, M, K, n_vtiles, epi, s);
  const int ntx = (n_vtiles + 7) / 8, ldp = ntx * 128;
  int ks = splitk_plan<T>(M, K, n_vtiles);
  if (!scratch || scratch_bytes < splitk_scratch_bytes<T>(M, K, n_vtiles)) ks = 1;
  dim3 grid(ntx, (M + 127) / 128, ks);
  gemm_tiled_kernel<T, AS, Epi><<<grid, 256, 0, s>>>(A, lda, arows, M, K, epi, K / ks, ks > 1 ? scratch : nullptr,
                                                     ldp);
  if (ks > 1) {
    const size_t n = static_cast<size_t>(M) * ldp;
    gemm_splitk_epilogue_kernel<Epi><<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(scratch, M, ldp, ks,
                                                                                          n_vtiles, epi);
  }
  return hipGetLastError();
}

}  // namespace dflash
