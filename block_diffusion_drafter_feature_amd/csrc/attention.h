// Block attention of the drafted block over the injected context.
//
// The 16 block rows of sequence b attend to cache rows 0..L_b-1 and to the 16
// block rows themselves, with no mask among them (bidirectional in the block,
// full over the context; cache rows >= L_b are never read into the result).
//
// Work split: one work-group of four waves per (split s, kv head, sequence).  The
// context rows of a sequence are cut into SC splits of whole 64-key tiles; the last of
// the S splits takes the 16 block keys (alone when SC = S - 1).  Each wave owns one query head of the GQA
// group (16 query rows); with G < 4 heads per kv head, the 4/G waves of a head
// share its 32-key slabs round-robin and are merged through LDS at the end.
//
// K/V streaming: the work-group stages each 64-key tile of K and V^T through LDS.
// Every thread fetches its share of the tile as 16-byte chunks (a wave reads whole
// cache rows, fully coalesced) into registers two tiles ahead, then writes them to
// a double-buffered LDS tile in the order the matrix cores read them:
//   K rows in "fragment order": LDS row 32j + 16t + r holds the key of S^T row r of
//     16-key tile t in slab j, so a fragment read is 16 consecutive LDS rows;
//   V^T rows by dim (keys contiguous), padded by 16 bytes against bank conflicts.
// Out-of-range chunks are fetched through buffer loads with an offset past the
// buffer's end, which return zeros without touching memory, so every thread issues
// the same loads every iteration.  V chunks past the context end are zeroed (the
// cache may hold anything there, and 0 * NaN would poison the sum).
//
// Per 32-key slab, per wave (matrix cores, operands from LDS):
//   S^T[key, q] = K Q^T: A = 16 key rows of K, B = Q^T (in registers).  The two 16-key
//     tiles of a slab use a permuted key order so that lane group g ends up holding
//     keys 8g..8g+7 of the slab for its query column -- exactly the B-operand layout of
//   O^T[dim, q] += V^T P^T: A = V^T (8 consecutive keys per lane), B = P^T straight
//     from the S^T registers.
// Online softmax in base 2 with a per-query reference point and running sum; the reference
// moves only when a score passes it by more than 2^8, so the running output is rarely
// rescaled.  With S == 1 the kernel writes the normalised output; otherwise each split
// writes (O, m, l) partials that attn_combine_kernel merges in split order (deterministic).
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
  float* part_o;     // [B][Hkv][S][G][16][hd]   (S > 1)
  float* part_ml;    // [B][Hkv][S][G][16][2]
  T* out;            // [B*16][H*hd]             (S == 1)
  int H, Hkv, cap, S;
  int B;             // sequences (the split length follows the longest context)
  int bs;            // block rows that are keys (dynamic block size); rows >= bs are padding
  float scale_log2;  // log2(e) / sqrt(hd)
  int SC;            // context splits: S, or S - 1 when the last split holds only the block keys
};

// LDS tile geometry (elements of T)
template <typename T, int HD>
struct AttnTile {
  static constexpr int TK = 64;                        // keys per tile
  static constexpr int CE = 16 / sizeof(T);            // elements per 16-byte chunk
  static constexpr int KSTR = HD + CE;                 // K tile row stride
  static constexpr int VSTR = TK + CE;                 // V^T tile row stride
  static constexpr int KCH = TK * HD / CE;             // chunks per K tile
  static constexpr int VCH = HD * TK / CE;             // chunks per V^T tile
  static constexpr int STAGE = TK * KSTR + HD * VSTR;  // elements per buffer
};

// zero the elements >= n (0 <= n < 16 / esize) of a 16-byte chunk
template <typename T>
__device__ __forceinline__ u32x4_t keep_first(u32x4_t v, int n) {
  if (sizeof(T) == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = j < n ? v[j] : 0u;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t m = (2 * j < n ? 0x0000ffffu : 0u) | (2 * j + 1 < n ? 0xffff0000u : 0u);
      v[j] &= m;
    }
  }
  return v;
}

// Keys per split: the longest context of the batch (clamped to cap) over the SC context
// splits, rounded up to whole tiles.  With SC = S - 1 the last split gets no context and
// holds only the block's 16 keys, so no work-group has a second memory round trip (the
// block keys) after its context tiles; with SC = S the last split takes both.  Computed
// alike by the attention and the combine kernels.
__device__ __forceinline__ int split_chunk(const int32_t* ctx_len, int B, int cap, int SC, int tk) {
  int lmax = 0;
  for (int i = 0; i < B; ++i) lmax = max(lmax, min(max(ctx_len[i], 0), cap));
  return max(tk, ((lmax + SC - 1) / SC + tk - 1) / tk * tk);
}

template <typename T, int HD, int G>
__global__ __launch_bounds__(256, 2) void block_attn_kernel(AttnArgs<T> a) {
  typedef Frag<T> F;
  typedef typename F::type frag_t;
  typedef AttnTile<T, HD> TL;
  constexpr int NT = 256;
  constexpr int KW = 4 / G;          // waves per head
  constexpr int KS = HD / 32;        // fragments along head_dim
  constexpr int DT = HD / 16;        // 16-dim output tiles
  constexpr int NK = TL::KCH / NT;   // K chunks per thread per tile
  constexpr int NV = TL::VCH / NT;   // V^T chunks per thread per tile
  constexpr int CPR = HD / TL::CE;   // chunks per K row
  constexpr int CPV = TL::TK / TL::CE;
  static_assert(TL::KCH % NT == 0 && TL::VCH % NT == 0, "tile must split evenly over the work-group");
  constexpr float kSlack = 8.f;     // log2 headroom of the softmax weights over the reference point
  static_assert(KW == 1 || (KW - 1) * G * 16 * (HD + 4) * 4 + KW * G * 16 * 8 <= 2 * TL::STAGE * sizeof(T),
                "wave merge must fit in the tile buffers");
  __shared__ __align__(16) T lds[2 * TL::STAGE];

  const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, lg = lane >> 4;
  const int hl = wave % G, kq = wave / G, head = kvh * G + hl;
  const int Hkv = a.Hkv, cap = a.cap, S = a.S;

  int L = a.ctx_len[b];
  L = L < 0 ? 0 : (L > cap ? cap : L);
  // every sequence of the batch is cut into chunks of the same length (the longest context
  // over S), so a ragged batch spreads its long contexts over more work-groups; a split
  // with no context keys has no work unless it is the last (the block's own keys)
  const int chunk = split_chunk(a.ctx_len, a.B, cap, a.SC, TL::TK);
  const int kbeg = min(L, s * chunk);
  const int kend = min(L, kbeg + chunk);
  if (kbeg == kend && s != S - 1) return;
  const int ntiles = (kend - kbeg + TL::TK - 1) / TL::TK;

  // query fragments of this wave's head
  frag_t qf[KS];
  {
    const T* qp = a.q + (static_cast<size_t>(b * 16 + r16) * a.H + head) * HD + lg * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = F::load(qp + ks * 32);
  }
  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mrow = -INFINITY, lsum = 0.f;

  // one 32-key slab: kf = K fragments of its two 16-key tiles, vf = V^T fragments
  auto slab = [&](const frag_t (&kf)[2][KS], const frag_t (&vf)[DT], int nvalid) {
    f32x4_t st[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      st[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) st[t] = F::mma(st[t], kf[t][ks], qf[ks]);
    }
    if (nvalid < 32) {   // a tail slab (wave-uniform): keys past the end get no weight
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (8 * lg + 4 * t + i >= nvalid) st[t][i] = -INFINITY;
    }
    // the raw maximum scaled once: x -> x * scale (scale > 0) preserves the order
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, st[t][i]);
    mx = max_lane_groups(mx) * a.scale_log2;
    // The softmax's reference point mrow moves only when a score passes it by more than
    // kSlack (base 2), or on the first slab; any reference gives the same normalised result,
    // and the weights exp2(s - mrow) stay <= 2^kSlack.  With no lane moving (wave-uniform),
    // the rescaling of the running sums is skipped altogether.
    const float mref = mx > mrow + kSlack ? mx : mrow;
    if (__ballot(mref != mrow)) {
      const float corr = __builtin_amdgcn_exp2f(mrow - mref);   // 0 on the first slab, 1 where unmoved
      lsum *= corr;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= corr;
      mrow = mref;
    }
    float sv[8], ps = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[4 * t + i] = __builtin_amdgcn_exp2f(fmaf(st[t][i], a.scale_log2, -mrow));
        ps += sv[4 * t + i];
      }
    lsum += ps;
    const frag_t pf = F::from_floats(sv);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = F::mma(o[dt], vf[dt], pf);
  };

  // ---- context tiles through LDS
  const size_t kv_base = static_cast<size_t>(b) * Hkv + kvh;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.kc + kv_base * cap * HD, static_cast<uint32_t>(cap) * HD * sizeof(T));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.vtc + kv_base * HD * cap, static_cast<uint32_t>(cap) * HD * sizeof(T));
  constexpr uint32_t kOut = 0x80000000u;   // past every buffer's end: loads return zero

  auto gload = [&](u32x4_t (&ck)[NK], u32x4_t (&cv)[NV], int tile) {
    const int kb0 = kbeg + tile * TL::TK;
#pragma unroll
    for (int p = 0; p < NK; ++p) {
      const int e = tid + p * NT, key = e / CPR, c = e % CPR;
      const uint32_t off = static_cast<uint32_t>((kb0 + key) * HD + c * TL::CE) * sizeof(T);
      ck[p] = __builtin_amdgcn_raw_buffer_load_b128(rk, kb0 + key < kend ? off : kOut, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < NV; ++p) {
      const int e = tid + p * NT, dim = e / CPV, c = e % CPV;
      const uint32_t off = static_cast<uint32_t>(dim * cap + kb0 + c * TL::CE) * sizeof(T);
      cv[p] = __builtin_amdgcn_raw_buffer_load_b128(rv, kb0 + c * TL::CE < kend ? off : kOut, 0, 0);
    }
  };
  auto lstore = [&](T* st, const u32x4_t (&ck)[NK], const u32x4_t (&cv)[NV], int tile) {
    const int kb0 = kbeg + tile * TL::TK;
#pragma unroll
    for (int p = 0; p < NK; ++p) {
      const int e = tid + p * NT, key = e / CPR, c = e % CPR;
      const int kk = key & 31;
      const int row = (key & 32) + 16 * ((kk >> 2) & 1) + 4 * (kk >> 3) + (kk & 3);
      *reinterpret_cast<u32x4_t*>(st + row * TL::KSTR + c * TL::CE) = ck[p];
    }
    T* sv = st + TL::TK * TL::KSTR;
    if (kb0 + TL::TK <= kend) {   // a whole tile (work-group-uniform)
#pragma unroll
      for (int p = 0; p < NV; ++p) {
        const int e = tid + p * NT, dim = e / CPV, c = e % CPV;
        *reinterpret_cast<u32x4_t*>(sv + dim * TL::VSTR + c * TL::CE) = cv[p];
      }
    } else {
#pragma unroll
      for (int p = 0; p < NV; ++p) {
        const int e = tid + p * NT, dim = e / CPV, c = e % CPV;
        const int nv = kend - (kb0 + c * TL::CE);
        *reinterpret_cast<u32x4_t*>(sv + dim * TL::VSTR + c * TL::CE) = nv >= TL::CE ? cv[p] : keep_first<T>(cv[p], nv);
      }
    }
  };
  auto compute = [&](const T* st, int tile) {
    const int kb0 = kbeg + tile * TL::TK;
    const T* sv = st + TL::TK * TL::KSTR;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int nvalid = kend - (kb0 + 32 * j);
      if (nvalid <= 0 || (2 * tile + j) % KW != kq) continue;
      frag_t kf[2][KS], vf[DT];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[t][ks] = F::load(st + (32 * j + 16 * t + r16) * TL::KSTR + ks * 32 + lg * 8);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) vf[dt] = F::load(sv + (dt * 16 + r16) * TL::VSTR + 32 * j + lg * 8);
      slab(kf, vf, nvalid);
    }
  };

  if (ntiles > 0) {
    T* buf0 = lds;
    T* buf1 = lds + TL::STAGE;
    u32x4_t k0[NK], v0[NV], k1[NK], v1[NV];
    gload(k0, v0, 0);
    __builtin_amdgcn_sched_barrier(0);   // keep tile 0's loads ahead of tile 1's
    gload(k1, v1, 1);
    // Each pass stores a landed tile, then fetches the tile two ahead into the same
    // registers before computing; every tile's loads stay in flight over two compute
    // phases.  The loop has a single exit at its head, so the loads are issued in the same
    // order on every path into it (tile 0 before tile 1 here) and only the older tile is
    // waited for.  A tile past the
    // end (odd count) reads zeros and computes nothing.
    for (int i = 0; i < ntiles; i += 2) {
      lstore(buf0, k0, v0, i);
      __syncthreads();
      gload(k0, v0, i + 2);
      compute(buf0, i);
      lstore(buf1, k1, v1, i + 1);
      __syncthreads();
      gload(k1, v1, i + 3);
      compute(buf1, i + 1);
    }
  }

  // ---- the block's own 16 keys (last split; the first wave of each head)
  if (s == S - 1 && kq == 0) {
    const int krow0 = 8 * (r16 >> 2) + (r16 & 3);
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
    slab(kf, vf, a.bs);   // padding rows of a smaller block are no keys
  }

  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);

  // ---- merge the waves of a head (fixed order kq = 0..KW-1)
  if (KW > 1) {
    constexpr int MST = HD + 4;
    float* mo = reinterpret_cast<float*>(lds);
    float* ml = mo + (KW - 1) * G * 16 * MST;
    __syncthreads();   // every wave is done with the tile buffers
    if (kq > 0) {
      float* p = mo + ((kq - 1) * G + hl) * 16 * MST + r16 * MST + 4 * lg;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4_t*>(p + dt * 16) = o[dt];
    }
    if (lg == 0) {
      ml[((kq * G + hl) * 16 + r16) * 2 + 0] = mrow;
      ml[((kq * G + hl) * 16 + r16) * 2 + 1] = lsum;
    }
    __syncthreads();
    if (kq == 0) {
      float M = mrow;
#pragma unroll
      for (int k = 1; k < KW; ++k) M = fmaxf(M, ml[((k * G + hl) * 16 + r16) * 2]);
      if (M != -INFINITY) {
        const float w0 = exp2f(mrow - M);
        float l = lsum * w0;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= w0;
#pragma unroll
        for (int k = 1; k < KW; ++k) {
          const float mk = ml[((k * G + hl) * 16 + r16) * 2];
          const float wk = mk == -INFINITY ? 0.f : exp2f(mk - M);
          l += wk * ml[((k * G + hl) * 16 + r16) * 2 + 1];
          const float* p = mo + ((k - 1) * G + hl) * 16 * MST + r16 * MST + 4 * lg;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[dt] += wk * *reinterpret_cast<const f32x4_t*>(p + dt * 16);
        }
        mrow = M;
        lsum = l;
      }
    }
  }
  if (kq != 0) return;

  // ---- output (S == 1) or partials
  if (S == 1) {
    const float inv = 1.f / lsum;
    T* op = a.out + (static_cast<size_t>(b) * 16 + r16) * a.H * HD + head * HD + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) op[dt * 16 + i] = from_f<T>(o[dt][i] * inv);
  } else {
    const size_t prow = ((kv_base * S + s) * G + hl) * 16 + r16;
    float* po = a.part_o + prow * HD + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4_t*>(po + dt * 16) = o[dt];
    if (lg == 0) {
      a.part_ml[prow * 2 + 0] = mrow;
      a.part_ml[prow * 2 + 1] = lsum;
    }
  }
}

// Merge the S (>= 2) split partials of the block rows of one (sequence, head); write
// the attention output rounded to the storage type, [B*16][H*hd].
// Four waves per work-group = (4 / SG row groups) x (SG split groups).  Lane l owns 8
// dims of one query row; the wave of split group p takes splits p, p+SG, ..., at most
// NS of them, and issues all their loads at once.  Order of the sums (fixed): within
// a wave by increasing split, then split groups 0..SG-1.
// grid (16 / (rows per wave * 4 / SG), H, B), 256 threads.
constexpr int kCombineMaxSplits = 64;
template <typename T, int HD, int SG, int NS>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml, T* __restrict__ out,
                                                           int H, int Hkv, int S, const int32_t* __restrict__ ctx_len,
                                                           int B, int cap, int tk, int SC) {
  constexpr int LPR = HD / 8;     // lanes per row
  constexpr int RPW = 64 / LPR;   // rows per wave
  constexpr int RG = 4 / SG;      // row groups per work-group
  static_assert(RG * RPW <= 16 && 16 % (RG * RPW) == 0, "row groups must tile the 16 block rows");
  __shared__ float red_m[4][64];
  __shared__ float red[4][64][9];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, rg = w / SG, p = w % SG;
  const int q = (blockIdx.x * RG + rg) * RPW + lane / LPR, d0 = (lane % LPR) * 8;
  const int head = blockIdx.y, b = blockIdx.z;
  const int G = H / Hkv, kvh = head / G, hl = head % G;
  const size_t sstride = static_cast<size_t>(G) * 16;                                    // rows per split
  const size_t row0 = (static_cast<size_t>(b * Hkv + kvh) * S * G + hl) * 16 + q;        // split 0
  // splits that wrote partials: those holding context keys, and the last
  const int L = min(max(ctx_len[b], 0), cap);
  const int chunk = split_chunk(ctx_len, B, cap, SC, tk);
  const int nctx = (L + chunk - 1) / chunk;
  auto live = [&](int s) { return s < S && (s < nctx || s == S - 1); };
  float m[NS], l[NS];
  f32x4_t x0[NS], x1[NS];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int s = p + SG * i;
    m[i] = -INFINITY;
    l[i] = 0.f;
    if (live(s)) {
      const size_t r = row0 + s * sstride;
      m[i] = part_ml[r * 2];
      l[i] = part_ml[r * 2 + 1];
      x0[i] = *reinterpret_cast<const f32x4_t*>(part_o + r * HD + d0);
      x1[i] = *reinterpret_cast<const f32x4_t*>(part_o + r * HD + d0 + 4);
      mx = fmaxf(mx, m[i]);
    }
  }
  red_m[w][lane] = mx;
  __syncthreads();
  float M = red_m[rg * SG][lane];
#pragma unroll
  for (int k = 1; k < SG; ++k) M = fmaxf(M, red_m[rg * SG + k][lane]);
  float den = 0.f, acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    if (live(p + SG * i)) {
      const float wt = m[i] == -INFINITY ? 0.f : exp2f(m[i] - M);
      den += wt * l[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[j] += wt * x0[i][j];
        acc[4 + j] += wt * x1[i][j];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) red[w][lane][j] = acc[j];
  red[w][lane][8] = den;
  __syncthreads();
  if (p != 0) return;
  float o[9];
#pragma unroll
  for (int j = 0; j < 9; ++j) {
    o[j] = red[rg * SG][lane][j];
#pragma unroll
    for (int k = 1; k < SG; ++k) o[j] += red[rg * SG + k][lane][j];
  }
  const float inv = 1.f / o[8];
  T* op = out + (static_cast<size_t>(b) * 16 + q) * H * HD + head * HD + d0;
#pragma unroll
  for (int j = 0; j < 8; ++j) op[j] = from_f<T>(o[j] * inv);
}

}  // namespace dflash
