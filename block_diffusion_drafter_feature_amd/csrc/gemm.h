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
// Three kernels:
//  * gemm_skinny : M <= 16 (one drafted block) up to K < 16384, and M <= 64 when
//    gemm_pipe does not apply (fp32).  Weight
//    streaming: each work-group owns NT virtual tiles over the whole K; its NW
//    waves split K, stream their slice of W straight from HBM into registers
//    (16 B per lane per fragment, two register stages in flight) and reduce
//    through LDS in a fixed order.
//  * gemm_pipe   : bf16 operands (A in bf16), M > 16 (and M <= 16 with K >= 16384).  64/128/256 x 128 output tiles per
//    work-group of 2x2 or 4x2 waves; 64-wide K slabs stream from memory straight into a ring
//    of LDS slots with several slabs in flight; tile shape and split-K per GEMM shape.
//  * gemm_tiled  : M > 64 when gemm_pipe does not apply (fp32, or A given in fp32).
//    128x128 output tile per work-group, A and W tiles staged through LDS (register
//    prefetch of the next K slab while the matrix cores work on the current one), 2x2
//    waves of 64x64.
// All are deterministic (no atomics).
#pragma once

#include "common.h"
#include <limits.h>
#include <type_traits>

namespace dflash {

template <typename T, typename AS>
__device__ __forceinline__ typename Frag<T>::type load_a(const AS* p) {
  if constexpr (std::is_same<AS, T>::value) return Frag<T>::load(p);
  else return Frag<T>::load_f32(p);
}

// Epilogue of an output tile held in LDS: Ct[r][.] (row stride ldc) holds rows m_base + r
// (r < rows) and the 16 columns of virtual tiles vt0 .. vt0 + nvt - 1.  The per-row facts
// are worked out once per row; a tile whose stores run along m (Epi::colmajor) gives
// consecutive rows to consecutive threads.  Called by every thread of the work-group;
// rinfo holds >= rows entries (ROWS_READY: already filled by the caller, and visible to every
// thread); cols, when given, the per-tile facts of tiles vt0.. (Epi::Col).  Ends without a
// barrier (the caller syncs before reusing Ct).
template <class Epi, bool ROWS_READY = false, int NTH = 0>
__device__ __forceinline__ void epilogue_tile(const Epi& epi, const float* Ct, int ldc, int m_base, int rows,
                                              int vt0, int nvt, int M, const typename Epi::Row* rinfo_in,
                                              const typename ColOf<Epi>::type* cols = nullptr,
                                              float2* trig = nullptr) {
  // NTH: the work-group size when known at compile time (the element loops then have a known
  // trip count, so their loads can be issued ahead of the stores)
  const int nth = NTH > 0 ? NTH : static_cast<int>(blockDim.x), tid = threadIdx.x;
  typename Epi::Row* rinfo = const_cast<typename Epi::Row*>(rinfo_in);
  if constexpr (!ROWS_READY) {
    for (int r = tid; r < rows; r += nth) rinfo[r] = epi.row(m_base + r < M ? m_base + r : M - 1);
    __syncthreads();
  }
  const int per = rows * 16;
  if constexpr (HasRope<Epi>::value && HasCol<Epi>::value) {
    // rotary epilogue: (cos, sin) of every row and frequency pair once, then the elements
    if (cols && trig) {
      const int np = epi.rope_pairs();
      for (int e = tid; e < rows * np; e += nth) {
        const int r = e / np, j = e - r * np;
        float cs, sn;
        rope_cs(rinfo[r].pos, epi.rope_inv(j), &cs, &sn);
        trig[e] = make_float2(cs, sn);
      }
      __syncthreads();
      if (rows % 8 == 0) {
        // 8-wide items, 2 * rows per tile: a rotated tile's row halves (8 consecutive
        // dimensions, rotated against the other half) or a value tile's columns over 8
        // consecutive rows; each item is one 16-byte store
        const int ipt = 2 * rows, nhalf = rows / 8;
        // rotated tiles of whole heads (groups of 8 vtiles): items in the order (group, row,
        // half, vtile of the group), so 16 consecutive lanes write one row's 16 chunks of a
        // head, 256 contiguous bytes; otherwise vtile by vtile
        const bool byrow = nvt % 8 == 0 && epi.kind8(cols[0]) > 0;
        for (int it = tid; it < nvt * ipt; it += nth) {
          int v, sub;
          if (byrow) {
            const int g8 = it / (8 * ipt), rem = it - g8 * 8 * ipt;
            v = 8 * g8 + (rem & 7);
            sub = rem >> 3;
          } else {
            v = it / ipt;
            sub = it - v * ipt;
          }
          const typename Epi::Col& cf = cols[v];
          const int kind = epi.kind8(cf);
          float o[8];
          if (kind > 0) {
            const int r = sub >> 1, h = sub & 1;
            if (m_base + r >= M) continue;
            const float* a = Ct + r * ldc + v * 16 + 8 * h;
            const float* b = Ct + r * ldc + v * 16 + 8 * (1 - h);
            const float2* t = trig + r * np + 8 * cf.tt;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const float2 cs = t[k];
              o[k] = h == 0 ? a[k] * cs.x - b[k] * cs.y : a[k] * cs.x + b[k] * cs.y;
            }
            epi.store8_rot(cf, m_base + r, rinfo[r], h, o);
          } else if (kind == 0) {
            const int c = sub / nhalf, r0 = 8 * (sub - c * nhalf);
            if (m_base + r0 >= M) continue;
#pragma unroll
            for (int k = 0; k < 8; ++k) o[k] = Ct[(r0 + k) * ldc + v * 16 + c];
            epi.store8_val(cf, m_base + r0, rinfo + r0, c, o, M);
          }
        }
        return;
      }
      for (int v = 0; v < nvt; ++v) {
        const bool cm = epi.colmajor(vt0 + v);
        for (int e = tid; e < per; e += nth) {
          const int r = cm ? e % rows : e >> 4, c = cm ? e / rows : e & 15;
          const int m = m_base + r;
          if (m >= M) continue;
          const float* row = Ct + r * ldc;
          epi.apply(cols[v], m, rinfo[r], c, row[v * 16 + c], row[((v ^ Epi::PX) << 4) | (c ^ Epi::PC)], trig + r * np);
        }
      }
      return;
    }
  }
  for (int v = 0; v < nvt; ++v) {
    const int vt = vt0 + v;
    const bool cm = epi.colmajor(vt);
    if constexpr (HasCol<Epi>::value) {
      if (cols) {   // (passed by reference: read in place from shared memory)
        for (int e = tid; e < per; e += nth) {
          const int r = cm ? e % rows : e >> 4, c = cm ? e / rows : e & 15;
          const int m = m_base + r;
          if (m >= M) continue;
          const float* row = Ct + r * ldc;
          epi.apply(cols[v], m, rinfo[r], c, row[v * 16 + c], row[((v ^ Epi::PX) << 4) | (c ^ Epi::PC)]);
        }
        continue;
      }
    }
    {
      for (int e = tid; e < per; e += nth) {
        const int r = cm ? e % rows : e >> 4, c = cm ? e / rows : e & 15;
        const int m = m_base + r;
        if (m >= M) continue;
        const float* row = Ct + r * ldc;
        epi.apply(vt, m, rinfo[r], c, row[v * 16 + c], row[((v ^ Epi::PX) << 4) | (c ^ Epi::PC)]);
      }
    }
  }
}

// wait until at most N of this wave's memory loads are outstanding and its LDS accesses
// are done, then a work-group barrier that carries no memory fence
template <int N>
__device__ __forceinline__ void pipe_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
  asm volatile("s_barrier" ::: "memory");
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
  __shared__ typename Epi::Row rinfo[ROWS];
  epilogue_tile(epi, &tile[0][0], TW + 1, 0, ROWS, vt0, NT, M, rinfo);
}

// Persistent weight streaming (M <= 16, bf16, K = NW * 32 * KS): one work-group of NW
// waves per compute unit walks a contiguous range of 16-column tiles.  Each wave holds its
// K slice of A (16 rows x 32 KS) in registers for the whole launch, so the only memory
// traffic per tile is the weight stream itself (re-reading A for every tile from the
// caches costs as many load instructions as the weights at one tile per work-group).  Two
// register buffers of W alternate across tiles: the next tile's loads are in flight while
// the current one is consumed, reduced over the waves (fixed order, through LDS) and
// handed to the epilogue.  The barriers carry no memory fence, so tile loads stay in
// flight across them.  The per-row facts of the epilogue are worked out once (the rows do
// not change from tile to tile).  Plain per-element epilogues over one weight matrix
// (EpiStore, EpiLogits) apply each sum directly; the others go through an LDS tile that
// holds each output's partner (a RoPE pair in the tile; with Epi::PX the gate/up pair of
// two consecutive tiles, so ranges start at even tiles).
template <class Epi>
struct StreamPlain {
  static constexpr bool value = Epi::kDirect && Epi::PX == 0 && Epi::PC == 0;
};

// W8: the weights are E4M3 codes with a float32 scale after each row (plain epilogues only):
// each lane loads 16 codes per 64-wide k group and widens them to two bf16 fragments when
// the tile is consumed; A follows the same k order (see gemm_skinny_w8_kernel) and the row
// scale multiplies the tile's sums before the reduction.
template <typename T, int NW, int KS, class Epi, bool W8 = false>
__global__ __launch_bounds__(64 * NW) void gemm_stream_kernel(const T* __restrict__ A, int lda, int M, int n_vtiles,
                                                              Epi epi) {
  typedef Frag<T> F;
  typedef typename F::type frag_t;
  constexpr bool kPlain = StreamPlain<Epi>::value;
  static_assert(!W8 || (kPlain && KS % 2 == 0), "FP8 weights: plain epilogues, whole 64-wide k groups");
  struct W8Buf {
    u32x4_t v[KS / 2];
    float sc;
  };
  static_assert(Epi::PX == 0 || Epi::PX == 1, "partner tile: none or the pair");
  static_assert(NW * 64 >= 256, "one thread per output of a tile");
  __shared__ float red[2][NW][256];
  __shared__ float ct[2][16][17];
  __shared__ typename Epi::Row rinfo[16];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int k0 = wave * 32 * KS;
  const int units = Epi::PX ? n_vtiles / 2 : n_vtiles;
  const int t_beg = static_cast<int>(static_cast<long>(units) * blockIdx.x / gridDim.x) << Epi::PX;
  const int t_end = static_cast<int>(static_cast<long>(units) * (blockIdx.x + 1) / gridDim.x) << Epi::PX;

  // running top 16 of this work-group's columns per row (kTop16): list[p] is written by the
  // tiles of parity p; entries start as distinct empties (-inf, ids above every column)
  __shared__ float tl_v[Epi::kTop16 ? 2 : 1][16][16];
  __shared__ int tl_i[Epi::kTop16 ? 2 : 1][16][16];
  __shared__ float tc_v[Epi::kTop16 ? 2 : 1][16][16];
  if constexpr (Epi::kTop16) {
    if (threadIdx.x < 256) {
      tl_v[1][threadIdx.x >> 4][threadIdx.x & 15] = -INFINITY;
      tl_i[1][threadIdx.x >> 4][threadIdx.x & 15] = INT_MAX - 16 - (threadIdx.x & 15);
    }
    if (t_beg >= t_end) {   // no columns: an empty list
      if (threadIdx.x < 256) {
        const int r = threadIdx.x >> 4, j = threadIdx.x & 15;
        if (r < M) {
          const size_t o = (static_cast<size_t>(r) * gridDim.x + blockIdx.x) * 16 + j;
          epi.tk_v[o] = -INFINITY;
          epi.tk_i[o] = INT_MAX - 16 - j;
        }
      }
      return;
    }
  }
  if (t_beg >= t_end) return;

  // this wave's K slice of A, kept for every tile (rows past M read row 0; never stored)
  frag_t a[KS];
  if constexpr (W8) {
    const T* ap = A + static_cast<size_t>(r16 < M ? r16 : 0) * lda + k0 + 16 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a[ks] = F::load(ap + 64 * (ks >> 1) + 8 * (ks & 1));
  } else {
    const T* ap = A + static_cast<size_t>(r16 < M ? r16 : 0) * lda + g * 8 + k0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a[ks] = F::load(ap + 32 * ks);
  }
  if constexpr (!kPlain) {
    if (threadIdx.x < 16) rinfo[threadIdx.x] = epi.row(threadIdx.x < M ? threadIdx.x : M - 1);
    __syncthreads();
  }

  // W of tile vt through a buffer descriptor over its matrix; tiles past this range and
  // rows past the matrix read nothing (offset past the descriptor's end)
  auto load = [&](frag_t (&w)[KS], int vt) {
    __amdgpu_buffer_rsrc_t rw;
    uint32_t vo;
    if constexpr (kPlain) {
      const int wrows = epi.w.off[1], ldw = epi.w.K;
      const uint32_t wbytes = static_cast<uint32_t>(static_cast<size_t>(wrows) * ldw * sizeof(T));
      rw = make_rsrc(epi.w.p[0], wbytes);
      const int n = vt * 16 + r16;
      vo = (vt < t_end && n < wrows) ? static_cast<uint32_t>((static_cast<size_t>(n) * ldw + g * 8 + k0) * sizeof(T))
                                     : wbytes;
    } else {
      const int v = vt < t_end ? vt : t_beg;
      const T* base;
      uint32_t bytes;
      epi.wseg(v, base, bytes);
      rw = make_rsrc(base, bytes);
      const T* p = epi.wrow(v, r16);
      vo = (p && vt < t_end) ? static_cast<uint32_t>((p - base + g * 8 + k0) * sizeof(T)) : bytes;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) w[ks] = F::load_buf(rw, vo + 32 * ks * sizeof(T), 0);
  };
  // FP8 rows: 4096 codes then the row's scale; lane group g takes codes 16g..16g+15 of each
  // 64-wide group (tiles past the range and rows past the matrix read nothing)
  auto load8 = [&](auto& w, int vt) {
    if constexpr (W8) {
      const int wrows = epi.w.off[1];
      const uint32_t rowb = static_cast<uint32_t>(epi.w.K * sizeof(T));
      const uint32_t wbytes = static_cast<uint32_t>(static_cast<size_t>(wrows) * rowb);
      const __amdgpu_buffer_rsrc_t rw = make_rsrc(epi.w.p[0], wbytes);
      const int n = vt * 16 + r16;
      const uint32_t rb = (vt < t_end && n < wrows) ? static_cast<uint32_t>(n) * rowb : wbytes;
#pragma unroll
      for (int u = 0; u < KS / 2; ++u)
        w.v[u] = __builtin_amdgcn_raw_buffer_load_b128(rw, rb + k0 + 64 * u + 16 * g, 0, 0);
      w.sc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, rb + NW * 32 * KS, 0, 0));
    }
  };
  auto finish = [&](auto& w, int vt, int par) {
    f32x4_t acc{0.f, 0.f, 0.f, 0.f};
    if constexpr (W8) {
#pragma unroll
      for (int u = 0; u < KS / 2; ++u) {
        frag_t lo, hi;
        fp8x16_to_bf16(w.v[u], lo, hi);
        acc = F::mma(acc, a[2 * u], lo);
        acc = F::mma(acc, a[2 * u + 1], hi);
      }
      acc *= w.sc;
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = F::mma(acc, a[ks], w[ks]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) red[par][wave][lane * 4 + i] = acc[i];
    pipe_barrier<63>();
    const int e = threadIdx.x, l = e >> 2, i = e & 3;
    float sum = 0.f;
    if (e < 256) {
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) sum += red[par][w2][e];
    }
    if constexpr (Epi::kTop16) {
      // store the logits if asked, then merge this tile's 16 candidates of each row into the
      // running list: every entry's rank in the union (16 old + 16 new, all distinct keys)
      // is counted exactly, and the 16 best land in their places of the other list
      const int m = 4 * (l >> 4) + i, c = l & 15;
      if (e < 256) {
        if (epi.out && m < M) epi.apply(vt, m, typename Epi::Row{}, c, sum, 0.f);
        tc_v[par][m][c] = vt * 16 + c < epi.w.off[1] ? sum : -INFINITY;
      }
      pipe_barrier<63>();
      if (e < 256) {
        const int r = e >> 4, j = e & 15;
        auto nid = [&](int k) { return vt * 16 + k < epi.w.off[1] ? vt * 16 + k : INT_MAX - k; };
        const float ov = tl_v[par ^ 1][r][j], nv = tc_v[par][r][j];
        const int oi = tl_i[par ^ 1][r][j], ni = nid(j);
        int ro = j, rn = 0;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const float ck = tc_v[par][r][k], lk = tl_v[par ^ 1][r][k];
          const int cik = nid(k), lik = tl_i[par ^ 1][r][k];
          ro += better(ck, cik, ov, oi) ? 1 : 0;
          rn += (better(ck, cik, nv, ni) ? 1 : 0) + (better(lk, lik, nv, ni) ? 1 : 0);
        }
        if (ro < 16) {
          tl_v[par][r][ro] = ov;
          tl_i[par][r][ro] = oi;
        }
        if (rn < 16) {
          tl_v[par][r][rn] = nv;
          tl_i[par][r][rn] = ni;
        }
      }
    } else if constexpr (kPlain) {
      const int m = 4 * (l >> 4) + i;
      if (e < 256 && m < M) epi.apply(vt, m, typename Epi::Row{}, l & 15, sum, 0.f);
    } else {
      if (e < 256) ct[par][4 * (l >> 4) + i][l & 15] = sum;
      if (Epi::PX && !(vt & 1)) return;   // the gate tile waits for its up tile
      pipe_barrier<63>();
      if (e < 256) {
        const int u = Epi::PX ? vt - 1 : vt;   // the tile the epilogue is called for
        const bool cm = epi.colmajor(u);
        const int r = cm ? (e & 15) : (e >> 4), c = cm ? (e >> 4) : (e & 15);
        if (r < M) {
          if (Epi::PX) epi.apply(u, r, rinfo[r], c, ct[0][r][c], ct[1][r][c]);
          else epi.apply(u, r, rinfo[r], c, ct[par][r][c], ct[par][r][c ^ Epi::PC]);
        }
      }
    }
  };
  int vt = t_beg;
  if constexpr (W8) {
    W8Buf w0, w1;
    load8(w0, t_beg);
    load8(w1, t_beg + 1);
    for (; vt + 2 < t_end; vt += 2) {
      finish(w0, vt, 0);
      load8(w0, vt + 2);
      finish(w1, vt + 1, 1);
      load8(w1, vt + 3);
    }
    finish(w0, vt, 0);
    if (vt + 1 < t_end) finish(w1, vt + 1, 1);
  } else {
    frag_t w0[KS], w1[KS];
    load(w0, t_beg);
    load(w1, t_beg + 1);
    for (; vt + 2 < t_end; vt += 2) {
      finish(w0, vt, 0);
      load(w0, vt + 2);
      finish(w1, vt + 1, 1);
      load(w1, vt + 3);
    }
    finish(w0, vt, 0);
    if (vt + 1 < t_end) finish(w1, vt + 1, 1);
  }
  const int last_par = vt + 1 < t_end ? 1 : 0;
  if constexpr (Epi::kTop16) {
    pipe_barrier<63>();
    if (threadIdx.x < 256) {
      const int r = threadIdx.x >> 4, j = threadIdx.x & 15;
      if (r < M) {
        const size_t o = (static_cast<size_t>(r) * gridDim.x + blockIdx.x) * 16 + j;
        epi.tk_v[o] = tl_v[last_par][r][j];
        epi.tk_i[o] = tl_i[last_par][r][j];
      }
    }
  }
}

// FP8-weight variant (one drafted block: M <= 16, A in bf16).  W rows hold E4M3 codes
// followed by the row's float32 scale.  Each lane loads 16 codes, k = 16g .. 16g+15 of a
// 64-wide k group, and widens them to two bf16 fragments when the stage is consumed (not
// when it is loaded, so the loads of the next stage stay in flight); the A fragments
// follow the same k order (k-step 2u takes k 16g .. 16g+7 of group u, k-step 2u+1 takes
// 16g+8 .. 16g+15), so each product pairs equal k.  The row scale multiplies the
// accumulator before the fixed-order reduction.
template <typename T, int NT, int NW, int U, class Epi>
__global__ __launch_bounds__(64 * NW) void gemm_skinny_w8_kernel(const T* __restrict__ A, int lda,
                                                                 const int32_t* __restrict__ arows, int M, int K,
                                                                 Epi epi) {
  typedef Frag<T> F;
  typedef typename F::type frag_t;
  static_assert(U % 2 == 0, "k-steps come in pairs");
  constexpr int TW = 16 * NT, UG = U / 2;
  __shared__ float red[NW][NT * 256];
  __shared__ float tile[16][TW + 1];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int vt0 = blockIdx.x * NT;
  const int kw = K / NW;
  const int k0 = wave * kw;
  __amdgpu_buffer_rsrc_t rw[NT];
  uint32_t vw[NT];
  float sc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const T* base;
    uint32_t bytes;
    epi.wseg(vt0 + nt, base, bytes);
    rw[nt] = make_rsrc(base, bytes);
    const T* p = epi.wrow(vt0 + nt, r16);
    vw[nt] = p ? static_cast<uint32_t>((p - base) * sizeof(T)) + g * 16 + k0 : bytes;
    sc[nt] = fp8_row_scale(p, K);
  }
  const int ar = r16 < M ? (arows ? arows[r16] : r16) : (arows ? arows[0] : 0);
  const T* ap = A + static_cast<size_t>(ar) * lda + g * 16 + k0;

  f32x4_t acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  constexpr int STEP = 32 * U;   // K elements per register stage
  auto load = [&](u32x4_t (&w)[UG][NT], frag_t (&a)[U], int kb) {
#pragma unroll
    for (int u = 0; u < UG; ++u) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) w[u][nt] = __builtin_amdgcn_raw_buffer_load_b128(rw[nt], vw[nt] + 64 * u, kb, 0);
      a[2 * u] = F::load(ap + kb + 64 * u);
      a[2 * u + 1] = F::load(ap + kb + 64 * u + 8);
    }
  };
  auto mma = [&](u32x4_t (&w)[UG][NT], frag_t (&a)[U]) {
#pragma unroll
    for (int u = 0; u < UG; ++u)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        frag_t lo, hi;
        fp8x16_to_bf16(w[u][nt], lo, hi);
        acc[nt] = F::mma(acc[nt], a[2 * u], lo);
        acc[nt] = F::mma(acc[nt], a[2 * u + 1], hi);
      }
  };

  const int nst = kw / STEP;
  u32x4_t wc[UG][NT];
  frag_t ac[U];
  load(wc, ac, 0);
  for (int st = 1; st < nst; ++st) {
    u32x4_t wn[UG][NT];
    frag_t an[U];
    load(wn, an, st * STEP);
    mma(wc, ac);
#pragma unroll
    for (int u = 0; u < UG; ++u)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) wc[u][nt] = wn[u][nt];
#pragma unroll
    for (int u = 0; u < U; ++u) ac[u] = an[u];
  }
  mma(wc, ac);

#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][(nt * 64 + lane) * 4 + i] = acc[nt][i] * sc[nt];
  __syncthreads();
  for (int e = threadIdx.x; e < NT * 256; e += 64 * NW) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += red[w][e];
    const int i = e & 3, l = (e >> 2) & 63, nt = e >> 8;
    tile[4 * (l >> 4) + i][nt * 16 + (l & 15)] = s;
  }
  __shared__ typename Epi::Row rinfo[16];
  epilogue_tile(epi, &tile[0][0], TW + 1, 0, 16, vt0, NT, M, rinfo);
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
    __shared__ typename Epi::Row rinfo[64];
    epilogue_tile<Epi, false, 256>(epi, Ct, BN + 1, m0 + half * 64, 64, vt0, BN / 16, M, rinfo);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------
// pipelined large-tile GEMM (bf16 operands): direct global -> LDS loads
// ---------------------------------------------------------------------------------
// BM x BN output tile per work-group of four waves (2 x 2), each wave a (BM/2) x (BN/2)
// block of 16x16 matrix-core tiles.  The 64-wide K slabs go straight from memory into a
// ring of NS LDS slots (16-byte direct loads, no staging registers), so
// NS - 1 slabs are in flight while the matrix cores consume one.  The direct loads are
// issued as instructions the compiler does not track, so it adds no waits of its own for
// them: each step waits (vmcnt) for this wave's loads of the slab about to be read, then
// meets the other waves at a barrier without a memory fence, which leaves the loads of
// later slabs in flight.  The loop ends by draining every load.
// Slot layout: row r of a tile holds its 8 16-byte chunks (64 K values) with chunk c at
// position c ^ ((r >> 1) & 7), so the 16 rows of a fragment read hit 16 distinct bank
// groups.  A wave's direct load writes 1 KB = 8 rows; lane l fetches the chunk that
// belongs at position l & 7 of row l >> 3.
// epilogues with a four-column store (plain rows) or a four-output gate/up pair store
template <class Epi, class = void>
struct HasApply4 : std::false_type {};
template <class Epi>
struct HasApply4<Epi, std::void_t<decltype(Epi::kApply4)>> : std::integral_constant<bool, Epi::kApply4> {};
template <class Epi, class = void>
struct HasPair4 : std::false_type {};
template <class Epi>
struct HasPair4<Epi, std::void_t<decltype(Epi::kPair4)>> : std::integral_constant<bool, Epi::kPair4> {};

template <typename T, int STAGE, int I>
__device__ __forceinline__ T* pipe_slot() {
  __shared__ __attribute__((aligned(16))) T s[STAGE];
  return s;
}


template <typename T, int BM, int BN, int NS, class Epi, bool W8, int NWV>
__global__ __launch_bounds__(64 * NWV) void gemm_pipe_kernel(const T* __restrict__ A, int lda,
                                                             const int32_t* __restrict__ arows, int M, int K, Epi epi,
                                                             int tiles_m, int kslice, float* __restrict__ partial,
                                                             int ldp) {
  typedef Frag<T> F;
  typedef typename F::type frag_t;
  static_assert(sizeof(T) == 2, "bf16 operands");
  static_assert(NS >= 2 && NS <= 4, "ring of 2..4 slots");
  static_assert(NWV == 4 || NWV == 8, "2x2 or 4x2 waves");
  constexpr int WM = NWV / 2;                      // wave rows; 2 wave columns
  constexpr int TM = BM / (16 * WM), TN = BN / 32; // 16x16 tiles per wave
  // direct loads per thread per slab (W rows of 64 E4M3 codes are half as long)
  constexpr int LA = BM * 8 / (64 * NWV), LB = (W8 ? BN * 4 : BN * 8) / (64 * NWV);
  static_assert(LA * 64 * NWV == BM * 8 && LB * 64 * NWV == (W8 ? BN * 4 : BN * 8), "loads must tile the slab");
  constexpr int LPS = LA + LB;
  constexpr int STAGE = (BM + (W8 ? BN / 2 : BN)) * 64;      // T elements per slot
  constexpr int EPR = 32 * (BN + 1) * 4 <= STAGE * 2 ? 32 : 16;   // epilogue rows per LDS pass
  static_assert(EPR * (BN + 1) * 4 <= STAGE * 2, "epilogue pass must fit in one slot");
  static_assert((NS - 2) * LPS < 64, "vmcnt range");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  int mt = blockIdx.x % tiles_m, nt = blockIdx.x / tiles_m;
  if constexpr (BN == 256) {
    // large grids: work-groups are dealt to the 8 XCDs round-robin, so give each XCD a run of
    // consecutive tiles in groups of 2 row tiles x all column tiles (its L2 then serves each
    // A slab to the column tiles and each W slab to both row tiles; A is fetched from HBM
    // about once).  A bijection of the grid; 16384 x 4096 x 20480: 0.51 -> 0.52-0.53.
    const int n = gridDim.x;
    if (n % 8 == 0 && tiles_m % 2 == 0) {
      const int W = (blockIdx.x % 8) * (n / 8) + blockIdx.x / 8;
      const int gsz = 2 * (n / tiles_m), r = W % gsz;
      mt = (W / gsz) * 2 + r % 2;
      nt = r / 2;
    }
  }
  constexpr int WR = BM / WM;                      // rows per wave
  const int m0 = mt * BM, vt0 = nt * (BN / 16);

  // this lane's source chunk for each of its direct loads: LDS block (8 rows) j*NWV + wave,
  // row block*8 + lane/8, position lane%8 <- chunk (lane%8) ^ ((row >> 1) & 7).
  // A: byte offsets from A (rows past M clamped); W: row pointers (past the end: row 0).
  // W8: 16 rows of 4 chunks per LDS block, chunk c of row r at position c ^ ((r >> 2) & 3).
  uint32_t aoff[LA];
  const char* wsrc[LB];
  const T* w0 = epi.wrow(vt0, 0);
#pragma unroll
  for (int j = 0; j < LA; ++j) {
    const int row = (j * NWV + wave) * 8 + (lane >> 3);
    const int ck = (lane & 7) ^ ((row >> 1) & 7);
    const int m = m0 + row < M ? m0 + row : M - 1;
    aoff[j] = static_cast<uint32_t>((static_cast<size_t>(arows ? arows[m] : m) * lda + ck * 8) * sizeof(T));
  }
#pragma unroll
  for (int j = 0; j < LB; ++j) {
    if constexpr (W8) {
      const int row = (j * NWV + wave) * 16 + (lane >> 2);
      const int ck = (lane & 3) ^ ((row >> 2) & 3);
      const T* wr = epi.wrow(vt0 + row / 16, row % 16);
      wsrc[j] = reinterpret_cast<const char*>(wr ? wr : w0) + ck * 16;
    } else {
      const int row = (j * NWV + wave) * 8 + (lane >> 3);
      const int ck = (lane & 7) ^ ((row >> 1) & 7);
      const T* wr = epi.wrow(vt0 + row / 16, row % 16);
      wsrc[j] = reinterpret_cast<const char*>((wr ? wr : w0) + ck * 8);
    }
  }
  auto issue = [&](const T* slot, int k0) {
    const uint32_t base = lds_addr(slot);
    const char* ak = reinterpret_cast<const char*>(A + k0);
#pragma unroll
    for (int j = 0; j < LA; ++j) dma16(ak + aoff[j], base + (j * NWV + wave) * 1024);
#pragma unroll
    for (int j = 0; j < LB; ++j) dma16(wsrc[j] + k0 * (W8 ? 1 : sizeof(T)), base + (BM / 8 + j * NWV + wave) * 1024);
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int sw = (r16 >> 1) & 7;
  auto compute = [&](const T* slot) {
    const T* As = slot + (wm * WR + r16) * 64;
    const T* Bs = slot + (BM + wn * (BN / 2) + r16) * 64;
    frag_t af[2][TM], bf[2][TN];
    if constexpr (W8) {
      // k-step ks of lane group g covers k 16g + 8ks .. +7 (the order of the widened codes)
      const uint8_t* Bs8 = reinterpret_cast<const uint8_t*>(slot + BM * 64) + (wn * (BN / 2) + r16) * 64 +
                           ((g ^ ((r16 >> 2) & 3)) * 16);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int pos = ((2 * g + ks) ^ sw) * 8;
#pragma unroll
        for (int i = 0; i < TM; ++i) af[ks][i] = F::load(As + i * 16 * 64 + pos);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fp8x16_to_bf16(*reinterpret_cast<const u32x4_t*>(Bs8 + j * 16 * 64), bf[0][j], bf[1][j]);
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int pos = ((4 * ks + g) ^ sw) * 8;
#pragma unroll
        for (int i = 0; i < TM; ++i) af[ks][i] = F::load(As + i * 16 * 64 + pos);
#pragma unroll
        for (int j = 0; j < TN; ++j) bf[ks][j] = F::load(Bs + j * 16 * 64 + pos);
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = F::mma(acc[i][j], af[ks][i], bf[ks][j]);
  };

  const int kofs = blockIdx.y * kslice;
  const int KT = (partial ? kslice : K) / 64;
  auto kslab = [&](int t) { return kofs + (t < KT ? t : KT - 1) * 64; };   // past the end: re-read the last
  T* const s0 = pipe_slot<T, STAGE, 0>();
  T* const s1 = pipe_slot<T, STAGE, 1>();
  T* const s2 = pipe_slot<T, (NS > 2 ? STAGE : 8), 2>();
  T* const s3 = pipe_slot<T, (NS > 3 ? STAGE : 8), 3>();
  auto slot = [&](int i) { return i == 0 ? s0 : i == 1 ? s1 : i == 2 ? s2 : s3; };
#pragma unroll
  for (int i = 0; i < NS - 1; ++i) issue(slot(i), kslab(i));
  // the per-row facts of the epilogue, worked out once per tile while the first slabs load
  // (their loads are dependent global reads for some epilogues)
  // (and the per-tile facts: kernel-argument arrays indexed at run time are memory reads)
  constexpr bool kRows = !std::is_empty<typename Epi::Row>::value;
  __shared__ typename Epi::Row rows_all[kRows ? BM : 1];
  __shared__ typename ColOf<Epi>::type cols_all[HasCol<Epi>::value ? BN / 16 : 1];
  if constexpr (kRows) {
    if (!partial)
      for (int r = tid; r < BM; r += 64 * NWV) rows_all[r] = epi.row(m0 + r < M ? m0 + r : M - 1);
  }
  if constexpr (HasCol<Epi>::value) {
    if (!partial && tid >= 64 * NWV - BN / 16) cols_all[tid - (64 * NWV - BN / 16)] = epi.col(vt0 + tid - (64 * NWV - BN / 16));
  }
  for (int kt = 0; kt < KT; kt += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      if (kt + u < KT) {
        pipe_barrier<(NS - 2) * LPS>();                  // slab kt+u landed; slot (u-1) free
        issue(slot((u + NS - 1) % NS), kslab(kt + u + NS - 1));
        compute(slot(u));
      }
    }
  }
  pipe_barrier<0>();   // drain the tail re-reads before the slots are reused
  if constexpr (W8) {   // row scales of this lane's columns
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const float sc = fp8_row_scale(epi.wrow(vt0 + wn * (BN / 32) + j, r16), K);
#pragma unroll
      for (int i = 0; i < TM; ++i) acc[i][j] *= sc;
    }
  }

  if (partial) {
    float* pz = partial + static_cast<size_t>(blockIdx.y) * M * ldp;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + wm * WR + i * 16 + 4 * g + e;
          if (m < M) pz[static_cast<size_t>(m) * ldp + vt0 * 16 + wn * (BN / 2) + j * 16 + r16] = acc[i][j][e];
        }
    return;
  }
  // epilogue, EPR rows at a time through slot 0
  float* const Ct = reinterpret_cast<float*>(s0);
#pragma unroll
  for (int h = 0; h < BM / EPR; ++h) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r0 = wm * WR + i * 16 - h * EPR;
      if (r0 >= 0 && r0 < EPR) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) Ct[(r0 + 4 * g + e) * (BN + 1) + wn * (BN / 2) + j * 16 + r16] = acc[i][j][e];
      }
    }
    __syncthreads();
    const typename ColOf<Epi>::type* cols = HasCol<Epi>::value ? cols_all : nullptr;
    // (cos, sin) table of a rotary epilogue in slot 1, free after the main loop
    float2* trig = nullptr;
    if constexpr (HasRope<Epi>::value) {
      if (static_cast<size_t>(EPR) * epi.rope_pairs() * sizeof(float2) <= STAGE * sizeof(T)) trig = reinterpret_cast<float2*>(s1);
    }
    if constexpr (HasTileMax<Epi>::value) {
      // the LM head's plain fp32 rows: four columns per thread, one 16-byte store each
      const int ncol = epi.w.off[epi.w.n_seg], n0 = vt0 * 16;
      const bool vec = epi.ldo % 4 == 0 && (reinterpret_cast<uintptr_t>(epi.out) & 15) == 0;
      constexpr int C4 = BN / 4;
#pragma unroll
      for (int e0 = 0; e0 < EPR * C4; e0 += 64 * NWV) {
        const int e = e0 + tid, r = e / C4, c = (e % C4) * 4, m = m0 + h * EPR + r, n = n0 + c;
        if (e >= EPR * C4 || m >= M) continue;
        const float* sp = Ct + r * (BN + 1) + c;
        float* o = epi.out + static_cast<size_t>(m) * epi.ldo + n;
        if (vec && n + 4 <= ncol) {
          *reinterpret_cast<f32x4_t*>(o) = f32x4_t{sp[0], sp[1], sp[2], sp[3]};
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (n + k < ncol) o[k] = sp[k];
        }
      }
    } else if constexpr (HasApply4<Epi>::value) {
      // plain fp32 rows (EpiStore): four columns per thread
      const int ncol = epi.w.off[epi.w.n_seg];
      const bool v4 = epi.ldo % 4 == 0 && (reinterpret_cast<uintptr_t>(epi.out) & 15) == 0;
#pragma unroll
      for (int e0 = 0; e0 < EPR * (BN / 4); e0 += 64 * NWV) {
        const int e = e0 + tid, r = e / (BN / 4), c = (e % (BN / 4)) * 4, m = m0 + h * EPR + r, n = vt0 * 16 + c;
        if (e < EPR * (BN / 4) && m < M) epi.apply4(m, n, Ct + r * (BN + 1) + c, v4 && n + 4 <= ncol, ncol);
      }
    } else if constexpr (HasPair4<Epi>::value) {
      // SwiGLU: a tile holds gate/up vtile pairs (columns 32j..32j+15 and 32j+16..32j+31);
      // four consecutive outputs per thread
#pragma unroll
      for (int e0 = 0; e0 < EPR * (BN / 8); e0 += 64 * NWV) {
        const int e = e0 + tid, r = e / (BN / 8), q = e % (BN / 8), j = q >> 2, c = (q & 3) * 4;
        const int m = m0 + h * EPR + r;
        if (e < EPR * (BN / 8) && m < M) {
          const float* g = Ct + r * (BN + 1) + 32 * j + c;
          epi.apply_pair4(m, (vt0 >> 1) * 16 + 16 * j + c, g, g + 16);
        }
      }
    } else if constexpr (kRows) {
      epilogue_tile<Epi, true, 64 * NWV>(epi, Ct, BN + 1, m0 + h * EPR, EPR, vt0, BN / 16, M, rows_all + h * EPR, cols, trig);
    } else {
      __shared__ typename Epi::Row rinfo[EPR];
      epilogue_tile<Epi, false, 64 * NWV>(epi, Ct, BN + 1, m0 + h * EPR, EPR, vt0, BN / 16, M, rinfo, cols);
    }
    if constexpr (HasTileMax<Epi>::value) {
      // each row's maximum over every 128-column group of the tile (past the vocabulary:
      // excluded; groups wholly past it are not written); 64 * NWV / EPR threads per row,
      // TPG of them per group (consecutive lanes, reduced by lane permutations)
      constexpr int TPR = 64 * NWV / EPR, CPT = BN / TPR, NGR = BN / 128, TPG = TPR / NGR;
      static_assert(BN % 128 == 0 && TPR <= 64 && (TPR & (TPR - 1)) == 0 && CPT * TPR == BN && TPG * NGR == TPR,
                    "row max layout");
      if (epi.tmax) {
        const int r = tid / TPR, q = tid % TPR, ncol = epi.w.off[epi.w.n_seg], ngr = (ncol + 127) / 128;
        float mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
          const int col = q * CPT + k;
          if (vt0 * 16 + col < ncol) mx = fmaxf(mx, Ct[r * (BN + 1) + col]);
        }
        if constexpr (TPG <= 16) {
          mx = group_max<TPG>(mx);
        } else {
#pragma unroll
          for (int o = 1; o < TPG; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        }
        const int m = m0 + h * EPR + r, grp = vt0 / 8 + q / TPG;
        if (q % TPG == 0 && m < M && grp < ngr) epi.tmax[static_cast<size_t>(m) * ngr + grp] = mx;
      }
    }
    __syncthreads();
  }
}

// Split-K reduction for epilogues that need no per-row facts and store along n
// (Epi::kDirect): one thread per (row, column), partials summed in z order.
template <class Epi>
__global__ __launch_bounds__(256) void gemm_splitk_direct_kernel(const float* __restrict__ partial, int M, int ldp,
                                                                 int ks, int n_vtiles, Epi epi) {
  const size_t e = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= static_cast<size_t>(M) * ldp) return;
  const int m = static_cast<int>(e / ldp), col = static_cast<int>(e % ldp);
  const int vt = col >> 4, c = col & 15;
  if (vt >= n_vtiles) return;
  const int pcol = ((vt ^ Epi::PX) << 4) | (c ^ Epi::PC);
  const size_t zs = static_cast<size_t>(M) * ldp;
  const float* p = partial + static_cast<size_t>(m) * ldp;
  // every partial's load issued before the first add (one memory round trip, not ks)
  float pz[8], qz[8];
#pragma unroll
  for (int z = 0; z < 8; ++z) {
    pz[z] = z < ks ? p[z * zs + col] : 0.f;
    qz[z] = (Epi::PX || Epi::PC) && z < ks ? p[z * zs + pcol] : 0.f;
  }
  float v = 0.f, pv = 0.f;
#pragma unroll
  for (int z = 0; z < 8; ++z) {
    if (z < ks) {
      v += pz[z];
      pv += qz[z];
    }
  }
  for (int z = 8; z < ks; ++z) {
    v += p[z * zs + col];
    if (Epi::PX || Epi::PC) pv += p[z * zs + pcol];
  }
  epi.apply(vt, m, epi.row(m), c, v, pv);
}

// The same for plain rows (Epi::kApply4): four columns per thread, 16-byte partial loads.
template <class Epi>
__global__ __launch_bounds__(256) void gemm_splitk_direct4_kernel(const float* __restrict__ partial, int M, int ldp,
                                                                  int ks, Epi epi, int xcd_nb) {
  const size_t l4 = static_cast<size_t>(ldp / 4);
  int m, col;
  if (xcd_nb > 0) {
    // the partials of 128-column block cb were written on XCD cb % 8: work-group w (XCD w % 8)
    // takes 8 rows x 128 columns of such a block
    const int w = blockIdx.x, x8 = w % 8, j = w / 8, per = xcd_nb / 8;
    const int cb = x8 + 8 * (j % per), rg = j / per;
    m = rg * 8 + (threadIdx.x >> 5);
    col = cb * 128 + (threadIdx.x & 31) * 4;
    if (m >= M) return;
  } else {
    const size_t e = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    if (e >= static_cast<size_t>(M) * l4) return;
    m = static_cast<int>(e / l4);
    col = static_cast<int>(e % l4) * 4;
  }
  const int ncol = epi.w.off[epi.w.n_seg];
  if (col >= ncol) return;
  const size_t zs = static_cast<size_t>(M) * ldp;
  const float* p = partial + static_cast<size_t>(m) * ldp + col;
  f32x4_t pz[8];
#pragma unroll
  for (int z = 0; z < 8; ++z)
    pz[z] = z < ks ? *reinterpret_cast<const f32x4_t*>(p + z * zs) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t v = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int z = 0; z < 8; ++z)
    if (z < ks) v += pz[z];
  for (int z = 8; z < ks; ++z) v += *reinterpret_cast<const f32x4_t*>(p + z * zs);
  const float vv[4] = {v[0], v[1], v[2], v[3]};
  const bool vec = epi.ldo % 4 == 0 && (reinterpret_cast<uintptr_t>(epi.out) & 15) == 0 && col + 4 <= ncol;
  epi.apply4(m, col, vv, vec, ncol);
}

template <class Epi>
static void launch_splitk_epilogue(const float* partial, int M, int ldp, int ks, int n_vtiles, const Epi& epi,
                                   hipStream_t s, int xcd_nb = 0);

// Split-K reduction: sum the partial tiles in z order into an LDS block of 16 rows x 64
// columns (each thread four consecutive columns of one row: a wave reads four 256-byte row
// segments of every partial with 16-byte loads), then the epilogue.
// grid (ldp / 64, ceil(M / 16)), 256 threads.
template <class Epi>
__global__ __launch_bounds__(256) void gemm_splitk_epilogue_kernel(const float* __restrict__ partial, int M,
                                                                   int ldp, int ks, int n_vtiles, Epi epi,
                                                                   int xcd_nb) {
  __shared__ float Ct[16 * 65];
  __shared__ typename Epi::Row rinfo[16];
  int c0 = blockIdx.x * 64, m0 = blockIdx.y * 16;
  if (xcd_nb > 0) {
    // the partials of 128-column block cb were written on XCD cb % 8: the work-group of
    // dispatch index w (XCD w % 8) takes a 64-column half of such a block
    const int w = blockIdx.y * gridDim.x + blockIdx.x, x8 = w % 8, j = w / 8, per = xcd_nb / 8;
    const int cb = x8 + 8 * (j % per), half = (j / per) % 2;
    c0 = (2 * cb + half) * 64;
    m0 = (j / per / 2) * 16;
  }
  const int r = threadIdx.x >> 4, cc = (threadIdx.x & 15) * 4;
  // the rows' and tiles' facts first: their loads overlap the partial loads below
  __shared__ typename ColOf<Epi>::type cols[HasCol<Epi>::value ? 4 : 1];
  const int vt0 = c0 / 16, nvt = min(4, n_vtiles - vt0);
  if (threadIdx.x < 16) rinfo[threadIdx.x] = epi.row(m0 + threadIdx.x < M ? m0 + threadIdx.x : M - 1);
  if constexpr (HasCol<Epi>::value) {
    if (threadIdx.x >= 64 && threadIdx.x < 64 + nvt) cols[threadIdx.x - 64] = epi.col(vt0 + threadIdx.x - 64);
  }
  const size_t zs = static_cast<size_t>(M) * ldp;
  {
    const int m = m0 + r;
    f32x4_t v = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (m < M) {
      const float* p = partial + static_cast<size_t>(m) * ldp + c0 + cc;
      f32x4_t part[8];
#pragma unroll
      for (int z = 0; z < 8; ++z) part[z] = z < ks ? *reinterpret_cast<const f32x4_t*>(p + z * zs) : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int z = 0; z < 8; ++z) v += part[z];
      for (int z = 8; z < ks; ++z) v += *reinterpret_cast<const f32x4_t*>(p + z * zs);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) Ct[r * 65 + cc + e] = v[e];
  }
  __syncthreads();
  float2* trig = nullptr;
  if constexpr (HasRope<Epi>::value) {
    __shared__ float2 trig_s[16 * 64];
    if (epi.rope_pairs() <= 64) trig = trig_s;
  }
  epilogue_tile<Epi, true, 256>(epi, Ct, 65, m0, 16, vt0, nvt, M, rinfo, HasCol<Epi>::value ? cols : nullptr, trig);
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

// Pipelined-GEMM plan (bf16 operands, A in bf16, M > 16): tile shape, LDS ring depth and split-K
// factor, from measurements on MI355X.
//  * M <= 64 (weight streaming), or grids of fewer than 32 tiles of 128 x 128: 64 x 128
//    tiles, 3 slots; K split until the grid has >= 128 work-groups (>= 256 at M <= 16).
//  * M >= 256: 256 x 128 tiles, 3 slots (each weight tile is read by fewer work-groups, and
//    the grid moves fewer bytes per flop); when there are fewer than 128 of them, K split
//    (at most 8 ways, >= 16 slabs per split) until the grid reaches 256 work-groups.  Cold
//    sweeps at 256 rows (x 4096 K unless noted), against 128 x 128 tiles without the long
//    splits: gate/up 24576 wide 92 -> 75 us (unsplit; 2 splits 90 us), QKV 6144 wide 40 ->
//    30 us (4 splits), O 4096 wide 36 -> 26 us (4), K/V injection 10240 wide 54 -> 44 us
//    (2), down (K 12288) 56 -> 42 us (8), context fusion (K 20480) 83 -> 57 us (8).
//  * M >= 512 with at least 256 tiles of 256 x 256: 256 x 256 tiles, 2 slots (half the
//    bytes per flop of 256 x 128; warm, 16384 x 4096 x 20480: 0.41 -> 0.50 of the bf16
//    peak, 16384 x 10240 x 4096: 0.39 -> 0.45, 512 x 151936 x 4096: 0.34 -> 0.37).
//  * otherwise 128 x 128 tiles, 2 slots (two work-groups per compute unit); when there are
//    fewer than 256 tiles, K split until the grid has >= 512 work-groups with >= 16 slabs
//    (1024 K values) per split.
// Splits keep K / 64 divisible (the fp32 partials are read back while still in cache).
struct BigPlan {
  int bm, bn, ns, ks;
};
inline BigPlan big_plan(int M, int K, int n_vtiles) {
  const int N = n_vtiles * 16;
  auto split = [&](long tiles, long want, int min_slabs, int max_ks = 8) {
    int ks = 1;
    while (ks < max_ks && tiles * ks < want && (K / 64) % (2 * ks) == 0 && K / 64 / (2 * ks) >= min_slabs) ks *= 2;
    return ks;
  };
  const long t128 = static_cast<long>((M + 127) / 128) * ((N + 127) / 128);
  if (M <= 64 || t128 < 32) {
    const long tiles = static_cast<long>((M + 63) / 64) * ((N + 127) / 128);
    return {64, 128, 3, split(tiles, M <= 16 ? 256 : 128, 4)};
  }
  const long t256 = static_cast<long>((M + 255) / 256) * ((N + 127) / 128);
  if (M >= 512 && static_cast<long>((M + 255) / 256) * ((N + 255) / 256) >= 256) return {256, 256, 2, 1};
  if (M >= 256) return {256, 128, 3, t256 < 128 ? split(t256, 256, 16, 8) : 1};
  return {128, 128, 2, t128 >= 256 ? 1 : split(t128, 512, 16)};
}

// True when run_gemm takes the pipelined kernel without split-K at this shape (bf16 weights):
// its epilogue then sees whole 128-column tiles (EpiLogits row maxima).
inline bool pipe_unsplit(int M, int K, int n_vtiles) {
  return M > 16 && K % 64 == 0 && big_plan(M, K, n_vtiles).ks == 1;
}

template <typename T>
inline size_t splitk_scratch_bytes(int M, int K, int n_vtiles) {
  const int ks = splitk_plan<T>(M, K, n_vtiles);
  size_t b = ks > 1 ? static_cast<size_t>(ks) * M * (((n_vtiles + 7) / 8) * 128) * sizeof(float) : 0;
  if (std::is_same<T, bf16_t>::value && K % 64 == 0) {   // (an upper bound: also for GEMMs that take another path)
    const BigPlan p = big_plan(M, K, n_vtiles);
    const size_t ldp = static_cast<size_t>((n_vtiles * 16 + p.bn - 1) / p.bn) * p.bn;
    if (p.ks > 1) b = std::max(b, static_cast<size_t>(p.ks) * M * ldp * sizeof(float));
  }
  return b;
}

// Skinny launch configuration (measured on MI355X with cold weights, M = 16, bf16): K
// split over 4 waves with 16 k-steps per register stage; two tiles per wave (a gate/up
// pair for SwiGLU) when there are at least 192 such work-groups and K <= 8192, else one.
// LM head 269 -> 246 us, gate/up 48 -> 44 us, down 30.5 -> 29.3 us against 8 k-steps.
// At M = 32, 64 (fp32 only) shorter stages.  K must be a multiple of NW * 32 * U;
// smaller stages and splits are used when it is not.
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
  constexpr int U = MT >= 4 ? 2 : (MT == 2 ? 4 : 16);
  const bool wide = n_vtiles / 2 >= 192 && K <= 8192;
  bool ok = false;
  // very wide plain outputs (LM head, K/V injection): four tiles per wave at half the
  // stage depth keep the same bytes in flight with fewer registers (cold sweep: 151936 x
  // 4096, 249 -> 240 us)
  if (MT == 1 && !Epi::PX && n_vtiles >= 512) ok = try_skinny<T, AS, MT, 4, 4, 8>(A, lda, arows, M, K, n_vtiles, epi, s);
  // long K (the down projection, 4096 x 12288): sixteen waves of 4 k-steps per stage keep
  // more of a work-group's weight stream in flight (cold sweep: 32.9 -> 27.3 us)
  if (!ok && MT == 1 && !Epi::PX && K >= 8192 && !wide)
    ok = try_skinny<T, AS, MT, 1, 16, 4>(A, lda, arows, M, K, n_vtiles, epi, s);
  if (!ok && (wide || Epi::PX)) ok = try_skinny<T, AS, MT, 2, 4, U>(A, lda, arows, M, K, n_vtiles, epi, s);
  if (!ok && !Epi::PX && MT == 1) ok = try_skinny<T, AS, MT, 1, 4, U>(A, lda, arows, M, K, n_vtiles, epi, s);
  if (!ok && (wide || Epi::PX)) ok = try_skinny<T, AS, MT, 2, 4, (U > 8 ? 8 : U)>(A, lda, arows, M, K, n_vtiles, epi, s);
  if (!ok && !Epi::PX) ok = try_skinny<T, AS, MT, 1, 8, (U > 8 ? 8 : U)>(A, lda, arows, M, K, n_vtiles, epi, s);
  if (!ok && !Epi::PX) ok = try_skinny<T, AS, MT, 1, 8, 2>(A, lda, arows, M, K, n_vtiles, epi, s);
  if (!ok) ok = try_skinny<T, AS, MT, (Epi::PX ? 2 : 1), 4, 1>(A, lda, arows, M, K, n_vtiles, epi, s);
  if (!ok) ok = try_skinny<T, AS, MT, (Epi::PX ? 2 : 1), 2, 1>(A, lda, arows, M, K, n_vtiles, epi, s);
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

template <class Epi>
static void launch_splitk_epilogue(const float* partial, int M, int ldp, int ks, int n_vtiles, const Epi& epi,
                                   hipStream_t s, int xcd_nb) {
  if constexpr (HasApply4<Epi>::value) {
    if (xcd_nb > 0) {
      const unsigned nwg = static_cast<unsigned>(xcd_nb) * ((M + 7) / 8);
      gemm_splitk_direct4_kernel<Epi><<<nwg, 256, 0, s>>>(partial, M, ldp, ks, epi, xcd_nb);
      return;
    }
    const size_t n = static_cast<size_t>(M) * (ldp / 4);
    gemm_splitk_direct4_kernel<Epi><<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(partial, M, ldp, ks, epi, 0);
  } else if (Epi::kDirect) {
    const size_t n = static_cast<size_t>(M) * ldp;
    gemm_splitk_direct_kernel<Epi><<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(partial, M, ldp, ks,
                                                                                        n_vtiles, epi);
  } else {
    gemm_splitk_epilogue_kernel<Epi><<<dim3(ldp / 64, (M + 15) / 16), 256, 0, s>>>(partial, M, ldp, ks, n_vtiles, epi,
                                                                                  xcd_nb);
  }
}

template <typename T, int BM, int BN, int NS, bool W8, class Epi, int NWV = 4>
static hipError_t launch_pipe_shape(const T* A, int lda, const int32_t* arows, int M, int K, int n_vtiles,
                                    const Epi& epi, int ks, float* scratch, hipStream_t s) {
  const int tm = (M + BM - 1) / BM, tn = (n_vtiles * 16 + BN - 1) / BN, ldp = tn * BN;
  gemm_pipe_kernel<T, BM, BN, NS, Epi, W8, NWV><<<dim3(tm * tn, ks), 64 * NWV, 0, s>>>(
      A, lda, arows, M, K, epi, tm, K / ks, ks > 1 ? scratch : nullptr, ldp);
  // one row tile of 128-column tiles, dealt to the XCDs round-robin: tile nt's partials on XCD nt % 8
  const int xcd_nb = BN == 128 && tm == 1 && tn % 8 == 0 ? tn : 0;
  if (ks > 1) launch_splitk_epilogue(scratch, M, ldp, ks, n_vtiles, epi, s, xcd_nb);
  return hipGetLastError();
}

template <typename T, bool W8, class Epi>
static hipError_t launch_big(const T* A, int lda, const int32_t* arows, int M, int K, int n_vtiles, const Epi& epi,
                             hipStream_t s, float* scratch, size_t scratch_bytes) {
  BigPlan p = big_plan(M, K, n_vtiles);
  const size_t ldp = static_cast<size_t>((n_vtiles * 16 + p.bn - 1) / p.bn) * p.bn;
  if (p.ks > 1 && (!scratch || scratch_bytes < static_cast<size_t>(p.ks) * M * ldp * sizeof(float))) p.ks = 1;
  // 64- and 256-row tiles run 8 waves (two per SIMD: one issues matrix-core work while the
  // other waits on LDS); warm sweeps at 512 x 151936 x 4096: 1020 -> 826 us, and at
  // 64 x 24576 x 4096: 41.6 -> 35.6 us
  if (p.bm == 64)
    return launch_pipe_shape<T, 64, 128, 3, W8, Epi, 8>(A, lda, arows, M, K, n_vtiles, epi, p.ks, scratch, s);
  if (p.bm == 256 && p.bn == 256 && !W8)
    return launch_pipe_shape<T, 256, 256, 2, W8, Epi, 8>(A, lda, arows, M, K, n_vtiles, epi, p.ks, scratch, s);
  if (p.bm == 256)   // (FP8 weights keep 256 x 128 tiles)
    return launch_pipe_shape<T, 256, 128, 3, W8, Epi, 8>(A, lda, arows, M, K, n_vtiles, epi, p.ks, scratch, s);
  return launch_pipe_shape<T, 128, 128, 2, W8>(A, lda, arows, M, K, n_vtiles, epi, p.ks, scratch, s);
}

template <typename T, int NT, int NW, int U, class Epi>
static bool try_skinny_w8(const T* A, int lda, const int32_t* arows, int M, int K, int n_vtiles, const Epi& epi,
                          hipStream_t s) {
  if (K % (NW * 32 * U) || n_vtiles % NT) return false;
  gemm_skinny_w8_kernel<T, NT, NW, U, Epi><<<n_vtiles / NT, 64 * NW, 0, s>>>(A, lda, arows, M, K, epi);
  return true;
}

template <typename T, class Epi>
static hipError_t launch_skinny_w8(const T* A, int lda, const int32_t* arows, int M, int K, int n_vtiles,
                                   const Epi& epi, hipStream_t s) {
  const bool wide = n_vtiles / 2 >= 192 && K <= 8192;
  constexpr int NTP = Epi::PX ? 2 : 1;
  bool ok = false;
  // E4M3 rows are half as long: K over two waves gives each wave as many stages as the
  // bf16 kernel's four
  if (wide || Epi::PX) ok = try_skinny_w8<T, 2, 2, 16>(A, lda, arows, M, K, n_vtiles, epi, s);
  if (!ok && (wide || Epi::PX)) ok = try_skinny_w8<T, 2, 4, 16>(A, lda, arows, M, K, n_vtiles, epi, s);
  if (!ok && !Epi::PX) ok = try_skinny_w8<T, 1, 4, 16>(A, lda, arows, M, K, n_vtiles, epi, s);
  if (!ok) ok = try_skinny_w8<T, NTP, 4, 8>(A, lda, arows, M, K, n_vtiles, epi, s);
  if (!ok) ok = try_skinny_w8<T, NTP, 4, 2>(A, lda, arows, M, K, n_vtiles, epi, s);
  if (!ok) ok = try_skinny_w8<T, NTP, 1, 2>(A, lda, arows, M, K, n_vtiles, epi, s);
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

// Work-groups of the persistent streaming kernel: one per compute unit of the current
// device (asked of the runtime at each launch, so no state is kept between calls), never
// more than there are work units.
inline int stream_grid(int n_vtiles) {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  return n_vtiles < n ? n_vtiles : n;
}

// One drafted block against a wide weight stream (QKV, K/V injection, gate/up, LM head):
// run_gemm takes the persistent streaming kernel, A resident in registers (bf16 weights).
template <typename T, class Epi>
inline bool stream_ok(int M, int K, int n_vtiles, const int32_t* arows, const Epi& epi) {
  if (!std::is_same<T, bf16_t>::value) return false;
  bool ok = M >= 1 && M <= 16 && !arows && K == 8 * 32 * 16 && n_vtiles >= 384 && n_vtiles % (Epi::PX + 1) == 0;
  if constexpr (StreamPlain<Epi>::value)
    ok = ok && epi.w.n_seg == 1 && static_cast<size_t>(epi.w.off[1]) * epi.w.K * sizeof(T) < (size_t{1} << 32) - 4096;
  return ok;
}

// The LM head of one drafted block with the first top-16 stage in its epilogue: returns
// the number of per-work-group lists written to epi.tk_v / tk_i ([M][groups][16]), or 0
// when the streaming kernel does not apply or would use more than max_groups work-groups
// (nothing is launched then).
template <typename T>
static int run_lm_head_top16(const T* A, int lda, int M, int K, int n_vtiles, const EpiLogitsTop16<T>& epi,
                             int max_groups, hipStream_t s, bool w8 = false) {
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (!stream_ok<T>(M, K, n_vtiles, nullptr, epi)) return 0;
    const int groups = stream_grid(n_vtiles);
    if (groups > max_groups) return 0;
    if (w8)
      gemm_stream_kernel<T, 8, 16, EpiLogitsTop16<T>, true><<<groups, 512, 0, s>>>(A, lda, M, n_vtiles, epi);
    else
      gemm_stream_kernel<T, 8, 16, EpiLogitsTop16<T>><<<groups, 512, 0, s>>>(A, lda, M, n_vtiles, epi);
    return hipGetLastError() == hipSuccess ? groups : -1;
  } else {
    return 0;
  }
}

// n_vtiles: number of virtual 16-column tiles (multiple of 2 when Epi::PX == 1).
// K: multiple of 64.  scratch: split-K partials (>= splitk_scratch_bytes, or nullptr: no split).
// w8: W in FP8 storage (E4M3 rows with a float32 scale; the epilogue's row stride covers
// the K codes and the 16-byte scale field).  Supported with bf16 A, K a multiple of 64
// and the pipelined kernel's 2 GiB A span, through gemm_pipe or gemm_skinny_w8 (M <= 16).
template <typename T, typename AS, class Epi>
static hipError_t run_gemm(const AS* A, int lda, const int32_t* arows, int M, int K, int n_vtiles, const Epi& epi,
                           hipStream_t s, float* scratch = nullptr, size_t scratch_bytes = 0, size_t a_rows = 0,
                           bool w8 = false) {
  if (M <= 0 || n_vtiles <= 0) return hipSuccess;
  if constexpr (std::is_same<T, bf16_t>::value && std::is_same<AS, T>::value) {
    // gemm_pipe addresses A with 32-bit byte offsets: the rows A spans (M, or the a_rows of
    // the table that arows gathers from) must fit in 2 GiB
    const size_t span = arows ? a_rows : static_cast<size_t>(M);
    // (at M <= 16 only for long K, where its split-K streams the weights faster than
    // gemm_skinny: 16 x 4096 x 20480 cold, 44 -> 39 us)
    const bool pipe_ok = K % 64 == 0 && span > 0 && span * lda * sizeof(T) < (size_t{1} << 31);
    if (w8) {
      if (M <= 16 && K % 64 == 0) return launch_skinny_w8<T, Epi>(A, lda, arows, M, K, n_vtiles, epi, s);
      if (pipe_ok) return launch_big<T, true, Epi>(A, lda, arows, M, K, n_vtiles, epi, s, scratch, scratch_bytes);
      return hipErrorNotSupported;
    }
    if ((M > 16 || K >= 16384) && pipe_ok)
      return launch_big<T, false, Epi>(A, lda, arows, M, K, n_vtiles, epi, s, scratch, scratch_bytes);
  }
  if (w8) return hipErrorNotSupported;
  if constexpr (std::is_same<T, bf16_t>::value && std::is_same<AS, T>::value) {
    if (stream_ok<T>(M, K, n_vtiles, arows, epi)) {
      gemm_stream_kernel<T, 8, 16, Epi><<<stream_grid(n_vtiles >> Epi::PX), 512, 0, s>>>(A, lda, M, n_vtiles, epi);
      return hipGetLastError();
    }
  }
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
    launch_splitk_epilogue(scratch, M, ldp, ks, n_vtiles, epi, s);
  }
  return hipGetLastError();
}

}  // namespace dflash
