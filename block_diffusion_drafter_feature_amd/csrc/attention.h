// Block attention of the drafted block over the injected context.
//
// The 16 block rows of sequence b attend to cache rows 0..L_b-1 and to the 16
// block rows themselves, with no mask among them (bidirectional in the block,
// full over the context; cache rows >= L_b are never read into the result).
//
// Work split: one work-group per (split s, kv head, sequence); the context rows of
// a sequence are cut into S splits (multiples of 32 rows); the last split also
// takes the 16 block keys.  Each wave handles HW query heads of the GQA group (16
// rows each) so every K/V element it loads feeds 16*HW query rows.
//
// Per 32-key slab, per wave:
//   S^T[key, q] = K Q^T  on the matrix cores: A = 16 key rows of K (dims
//     contiguous, straight from HBM), B = Q^T (loaded once).  The two 16-key tiles
//     of a slab use a permuted key order so that lane group g ends up holding keys
//     8g..8g+7 of the slab for its query column -- exactly the B-operand layout of
//   O^T[dim, q] += V^T P^T: A = V^T (the cache stores V transposed, keys
//     contiguous, so lane (dim, g) reads 8 consecutive keys in one 16-byte load),
//     B = P^T straight from the S^T registers.  No LDS, no transposes.
// Online softmax in base 2 with per-query running max/sum; the per-lane partial
// sums are reduced once at the end.  Partials (O, m, l) per split are merged by
// attn_combine_kernel in a fixed order (deterministic).
#pragma once

#include "common.h"

namespace dflash {

template <typename T>
struct AttnArgs {
  const T* q;        // [B*16][H][hd]
  const T* kb;       // [B][Hkv][16][hd]
  const T* vbt;      // [B][Hkv][hd][16]
  const T* kc;       // [B][Hkv][cap][hd]
  const T* vtc;      // [B][Hkv][hd][cap]
  const int32_t* ctx_len;
  float* part_o;     // [B][Hkv][S][G][16][hd]
  float* part_ml;    // [B][Hkv][S][G][16][2]
  int H, Hkv, cap, S;
  float scale_log2;  // log2(e) / sqrt(hd)
};

template <typename T, int HD, int G, int HW>
__global__ __launch_bounds__(64 * (G / HW)) void block_attn_kernel(AttnArgs<T> a) {
  typedef Frag<T> F;
  typedef typename F::type frag_t;
  constexpr int KS = HD / 32;   // fragments along head_dim
  constexpr int DT = HD / 16;   // 16-dim output tiles
  const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, lg = lane >> 4;
  const int Hkv = a.Hkv, cap = a.cap, S = a.S;

  int L = a.ctx_len[b];
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int chunk = (((L + S - 1) / S) + 31) & ~31;
  const int kbeg = s * chunk;
  const int kend = min(L, kbeg + chunk);

  frag_t qf[HW][KS];
#pragma unroll
  for (int h = 0; h < HW; ++h) {
    const int head = kvh * G + wave * HW + h;
    const T* qp = a.q + (static_cast<size_t>(b * 16 + r16) * a.H + head) * HD + lg * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[h][ks] = F::load(qp + ks * 32);
  }
  f32x4_t o[HW][DT];
  float mrow[HW], lsum[HW];
#pragma unroll
  for (int h = 0; h < HW; ++h) {
    mrow[h] = -INFINITY;
    lsum[h] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[h][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // key of S^T row r in tile t of a slab: 8*(r/4) + 4*t + r%4
  const int krow0 = 8 * (r16 >> 2) + (r16 & 3);
  const size_t kv_base = static_cast<size_t>(b) * Hkv + kvh;

  // one 32-key slab: kf = K fragments of the two tiles, vf = V^T fragments, nvalid = keys < nvalid count
  auto slab = [&](const frag_t (&kf)[2][KS], const frag_t (&vf)[DT], int nvalid) {
#pragma unroll
    for (int h = 0; h < HW; ++h) {
      f32x4_t st[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        st[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) st[t] = F::mma(st[t], kf[t][ks], qf[h][ks]);
      }
      float sv[8];
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 8 * lg + 4 * t + i;
          const float v = key < nvalid ? st[t][i] * a.scale_log2 : -INFINITY;
          sv[4 * t + i] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(mrow[h], mx);
      const float corr = exp2f(mrow[h] - mnew);
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sv[e] = exp2f(sv[e] - mnew);
        ps += sv[e];
      }
      lsum[h] = lsum[h] * corr + ps;
      mrow[h] = mnew;
      const frag_t pf = F::from_floats(sv);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        o[h][dt] *= corr;
        o[h][dt] = F::mma(o[h][dt], vf[dt], pf);
      }
    }
  };

  // ---- context slabs of this split: the next slab's K/V loads are issued before the
  // current slab is processed (one carried register stage)
  const T* kcp = a.kc + kv_base * cap * HD;
  const T* vcp = a.vtc + kv_base * HD * cap;
  auto load_slab = [&](frag_t (&kf)[2][KS], frag_t (&vf)[DT], int kb0) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const T* kp = kcp + static_cast<size_t>(kb0 + krow0 + 4 * t) * HD + lg * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[t][ks] = F::load(kp + ks * 32);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vf[dt] = F::load(vcp + static_cast<size_t>(dt * 16 + r16) * cap + kb0 + 8 * lg);
  };
  auto run_slab = [&](const frag_t (&kf)[2][KS], frag_t (&vf)[DT], int kb0) {
    const int nvalid = kend - kb0;                     // > 0
    if (nvalid < 32) {
      uint32_t keep = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) keep |= (8 * lg + j < nvalid ? 1u : 0u) << j;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) vf[dt] = F::mask(vf[dt], keep);
    }
    slab(kf, vf, nvalid);
  };
  if (kbeg < kend) {
    frag_t kc[2][KS], vc[DT];
    load_slab(kc, vc, kbeg);
    for (int kb0 = kbeg; kb0 < kend; kb0 += 32) {
      if (kb0 + 32 < kend) {
        frag_t kn[2][KS], vn[DT];
        load_slab(kn, vn, kb0 + 32);
        run_slab(kc, vc, kb0);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) kc[t][ks] = kn[t][ks];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vc[dt] = vn[dt];
      } else {
        run_slab(kc, vc, kb0);
      }
    }
  }

  // ---- the block's own 16 keys (last split only)
  if (s == S - 1) {
    frag_t kf[2][KS], vf[DT];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int key = krow0 + 4 * t;
      const T* kp = a.kb + (kv_base * 16 + (key < 16 ? key : 0)) * HD + lg * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[t][ks] = key < 16 ? F::load(kp + ks * 32) : F::zero();
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      vf[dt] = lg < 2 ? F::load(a.vbt + (kv_base * HD + dt * 16 + r16) * 16 + 8 * lg) : F::zero();
    slab(kf, vf, 16);
  }

  // ---- partials
#pragma unroll
  for (int h = 0; h < HW; ++h) {
    float l = lsum[h];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int hl = wave * HW + h;
    const size_t pbase = ((kv_base * S + s) * G + hl) * 16;
    float* po = a.part_o + (pbase + r16) * HD;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) po[dt * 16 + 4 * lg + i] = o[h][dt][i];
    if (lg == 0) {
      a.part_ml[(pbase + r16) * 2 + 0] = mrow[h];
      a.part_ml[(pbase + r16) * 2 + 1] = l;
    }
  }
}

// Merge the S split partials of one query row (sequence b, head, block row q) in split
// order; write the attention output rounded to the storage type, [B*16][H*hd].
// grid (16, H, B), HD threads (one per output dim).
template <typename T, int HD>
__global__ __launch_bounds__(HD) void attn_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml, T* __restrict__ out,
                                                          int H, int Hkv, int S) {
  __shared__ float w[64];
  __shared__ float inv_den;
  const int q = blockIdx.x, head = blockIdx.y, b = blockIdx.z, dim = threadIdx.x;
  const int G = H / Hkv, kvh = head / G, hl = head % G;
  const size_t base = ((static_cast<size_t>(b) * Hkv + kvh) * S) * G * 16;   // split 0
  const size_t sstride = static_cast<size_t>(G) * 16;
  const size_t row = hl * 16 + q;
  if (threadIdx.x < 64) {
    // split weights: exp2(m_s - max m), computed by the first wave
    const int s = threadIdx.x;
    const float m = s < S ? part_ml[(base + s * sstride + row) * 2] : -INFINITY;
    const float l = s < S ? part_ml[(base + s * sstride + row) * 2 + 1] : 0.f;
    float M = m;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    const float ws = s < S ? exp2f(m - M) : 0.f;
    w[s] = ws;
    // fixed-order denominator: lane 0 sums the split terms in split order
    float den = 0.f;
    for (int t = 0; t < S; ++t) den += __shfl(ws * l, t, 64);
    if (s == 0) inv_den = 1.f / den;
  }
  __syncthreads();
  float num = 0.f;
  for (int s = 0; s < S; ++s) num += w[s] * part_o[(base + s * sstride + row) * HD + dim];
  out[(static_cast<size_t>(b) * 16 + q) * H * HD + head * HD + dim] = from_f<T>(num * inv_den);
}

}  // namespace dflash
