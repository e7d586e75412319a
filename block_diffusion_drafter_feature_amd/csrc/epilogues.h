// Epilogue functors of the GEMMs: where W rows come from and what happens to each
// output element.  Interface used by gemm.h:
//   PX, PC            partner of (virtual tile vt, column c) is (vt ^ PX, c ^ PC)
//   wrow(vt, c)       pointer to the W row feeding column c of virtual tile vt (nullptr: zero)
//   wseg(vt, b, n)    the weight matrix holding tile vt's rows: base b, n bytes (n = 0 when
//                     the tile is past the end); every row of a tile lies in one matrix
//   Row, row(m)       per-row facts the epilogue needs (owning sequence, position), worked
//                     out once per output row and shared by all its columns
//   colmajor(vt)      true when tile vt's outputs are contiguous along m (transposed
//                     stores): the kernels then hand consecutive rows to consecutive threads
//   kDirect           true when Row is empty and no tile is colmajor (plain per-element
//                     epilogues need no staging tile)
//   kTop16            the streaming LM head keeps per-work-group top-16 lists (EpiLogitsTop16)
//   apply(vt, m, row, c, v, partner)
//   Col, col(vt)      optional: per-tile facts (destination, kind) worked out once per virtual
//                     tile; the staged epilogues then call apply(col, m, row, c, v, partner)
//   kRope             optional: rotary epilogue; rope_pairs(), rope_inv(j) give the frequencies
//                     and apply(col, m, row, c, v, partner, cs_row) takes the row's (cos, sin)
//                     table (Row has pos); kind8(col) (1 rotated, 0 value, -1 none),
//                     store8_rot(col, m, row, half, v[8]) (8 consecutive dimensions of a row)
//                     and store8_val(col, m0, rows, c, v[8], M) (column c of 8 consecutive
//                     rows) store 8 finished values at once
#pragma once

#include "common.h"

#include <type_traits>

namespace dflash {

// Up to 16 weight matrices stacked along N.
template <typename T>
struct SegW {
  const T* p[16];
  int off[17];   // row offsets, off[n_seg] = total rows
  int n_seg;
  int K;
  __device__ __forceinline__ int find(int n) const {
    int s = 0;
    while (s + 1 < n_seg && n >= off[s + 1]) ++s;
    return s;
  }
};

// Rotary-pair column layout: the 16 columns of a tile are 8 dims of the first half
// of a head and their 8 partners of the second half.
__device__ __forceinline__ int rope_dim(int tt, int c, int hd) {
  return (c < 8) ? 8 * tt + c : hd / 2 + 8 * tt + (c - 8);
}

// ------------------------------------------------------------------ plain store / residual / sigmoid

enum StoreMode { STORE = 0, ADD = 1, SIGMOID = 2, SILU = 3 };

template <typename T>
struct EpiStore {
  SegW<T> w;
  float* out;
  int ldo;
  int mode;
  static constexpr int PX = 0, PC = 0;
  static constexpr bool kDirect = true;
  static constexpr bool kTop16 = false;
  __device__ __forceinline__ const T* wrow(int vt, int c) const {
    const int n = vt * 16 + c;
    if (n >= w.off[w.n_seg]) return nullptr;
    const int s = w.find(n);
    return w.p[s] + static_cast<size_t>(n - w.off[s]) * w.K;
  }
  __device__ __forceinline__ void wseg(int vt, const T*& b, uint32_t& n) const {
    const int r = vt * 16;
    if (r >= w.off[w.n_seg]) {
      b = w.p[0];
      n = 0;
      return;
    }
    const int s = w.find(r);
    b = w.p[s];
    n = static_cast<uint32_t>(static_cast<size_t>(w.off[s + 1] - w.off[s]) * w.K * sizeof(T));
  }
  struct Row {};
  __device__ __forceinline__ Row row(int) const { return Row{}; }
  __device__ __forceinline__ bool colmajor(int) const { return false; }
  __device__ __forceinline__ void apply(int vt, int m, const Row&, int c, float v, float) const {
    const int n = vt * 16 + c;
    if (n >= w.off[w.n_seg]) return;
    float* o = out + static_cast<size_t>(m) * ldo + n;
    if (mode == ADD) *o += v;
    else if (mode == SIGMOID) *o = 1.f / (1.f + expf(-v));
    else if (mode == SILU) *o = v / (1.f + expf(-v));
    else *o = v;
  }
  // four consecutive columns n..n+3 of row m at once (the staged epilogues), the same values
  // as apply() column by column; ncol = w.off[w.n_seg] and vec (one 16-byte access: the
  // four columns exist, ldo % 4 == 0, out 16-byte aligned) worked out by the caller
  static constexpr bool kApply4 = true;
  __device__ __forceinline__ void apply4(int m, int n, const float* v, bool vec, int ncol) const {
    float* o = out + static_cast<size_t>(m) * ldo + n;
    if (mode == STORE) {   // (uniform) the plain store: no transform to evaluate
      if (vec) {
        *reinterpret_cast<f32x4_t*>(o) = f32x4_t{v[0], v[1], v[2], v[3]};
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (n + k < ncol) o[k] = v[k];
      }
      return;
    }
    float r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (mode == SIGMOID) r[k] = 1.f / (1.f + expf(-v[k]));
      else if (mode == SILU) r[k] = v[k] / (1.f + expf(-v[k]));
      else r[k] = v[k];
    }
    if (vec) {
      f32x4_t x = f32x4_t{r[0], r[1], r[2], r[3]};
      if (mode == ADD) x += *reinterpret_cast<const f32x4_t*>(o);
      *reinterpret_cast<f32x4_t*>(o) = x;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (n + k < ncol) o[k] = mode == ADD ? o[k] + r[k] : r[k];
    }
  }
};

// LM-head logits: a plain fp32 store, kept as its own type so that the LM-head GEMM is a
// kernel of its own in profiles.  With tmax != nullptr the pipelined kernel (unsplit, 128-
// column tiles) also writes each row's maximum over every 128-column group of the logits,
// tmax[m][n / 128] (columns past the vocabulary excluded).
template <typename T>
struct EpiLogits : EpiStore<T> {
  float* tmax;
};
template <class Epi, class = void>
struct HasCol : std::false_type {};
template <class Epi>
struct HasCol<Epi, std::void_t<typename Epi::Col>> : std::true_type {};
// Epi::Col, or an empty stand-in for epilogues without per-tile facts
template <class Epi, bool = HasCol<Epi>::value>
struct ColOf {
  struct type {};
};
template <class Epi>
struct ColOf<Epi, true> {
  typedef typename Epi::Col type;
};

// Epilogues with rotary pairs (Epi::kRope): the staged epilogues may hand apply() a table of
// (cos, sin) per row and frequency, worked out once per row and pair instead of per element.
template <class Epi, class = void>
struct HasRope : std::false_type {};
template <class Epi>
struct HasRope<Epi, std::void_t<decltype(Epi::kRope)>> : std::integral_constant<bool, Epi::kRope> {};

// 8 consecutive values of T from floats: one 16-byte (bf16) or two (fp32) stores when p is
// aligned for them, else element by element
template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&o)[8]) {
  if ((reinterpret_cast<uintptr_t>(p) & (8 * sizeof(T) - 1)) == 0) {
    if constexpr (sizeof(T) == 2) {
      u32x4_t w;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        w[k] = static_cast<uint32_t>(from_f<T>(o[2 * k])) | (static_cast<uint32_t>(from_f<T>(o[2 * k + 1])) << 16);
      *reinterpret_cast<u32x4_t*>(p) = w;
    } else {
      reinterpret_cast<f32x4_t*>(p)[0] = f32x4_t{o[0], o[1], o[2], o[3]};
      reinterpret_cast<f32x4_t*>(p)[1] = f32x4_t{o[4], o[5], o[6], o[7]};
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) p[k] = from_f<T>(o[k]);
  }
}

template <class Epi>
struct HasTileMax {
  static constexpr bool value = false;
};
template <typename T>
struct HasTileMax<EpiLogits<T>> {
  static constexpr bool value = true;
};

// LM head of one drafted block with the first top-16 stage folded in (streaming kernel
// only): every work-group keeps the running top 16 of its columns for each row (value
// descending, then column ascending) and writes them to tk_v / tk_i [M][groups][16]; the
// logits themselves are stored only when `out` is non-null.
template <typename T>
struct EpiLogitsTop16 : EpiStore<T> {
  float* tk_v;
  int32_t* tk_i;
  static constexpr bool kTop16 = true;
};

// ------------------------------------------------------------------ block Q/K/V with RoPE

template <typename T>
struct EpiQKV {
  const T* wq;
  const T* wk;
  const T* wv;
  int K, H, Hkv, hd;
  RopeFreq rf;             // inverse rotary frequencies
  const int32_t* ctx_len;  // [B]
  T* q;                    // [M][H][hd]
  T* kb;                   // [B][Hkv][16][hd]
  T* vbt;                  // [B][Hkv][hd][16]
  static constexpr int PX = 0, PC = 8;
  static constexpr bool kDirect = false;
  static constexpr bool kTop16 = false;
  // virtual tiles: H*hd/16 query tiles, Hkv*hd/16 key tiles (both RoPE-paired), Hkv*hd/16 value tiles
  __device__ __forceinline__ const T* wrow(int vt, int c) const {
    const int tq = H * hd / 16, tk = Hkv * hd / 16, tph = hd / 16;
    if (vt < tq) return wq + static_cast<size_t>((vt / tph) * hd + rope_dim(vt % tph, c, hd)) * K;
    vt -= tq;
    if (vt < tk) return wk + static_cast<size_t>((vt / tph) * hd + rope_dim(vt % tph, c, hd)) * K;
    vt -= tk;
    if (vt < tk) return wv + static_cast<size_t>(vt * 16 + c) * K;
    return nullptr;
  }
  __device__ __forceinline__ void wseg(int vt, const T*& b, uint32_t& n) const {
    const int tq = H * hd / 16, tk = Hkv * hd / 16;
    const size_t rb = static_cast<size_t>(K) * sizeof(T);
    if (vt < tq) { b = wq; n = static_cast<uint32_t>(H * hd * rb); }
    else if (vt < tq + tk) { b = wk; n = static_cast<uint32_t>(Hkv * hd * rb); }
    else if (vt < tq + 2 * tk) { b = wv; n = static_cast<uint32_t>(Hkv * hd * rb); }
    else { b = wq; n = 0; }
  }
  struct Row {
    int pos;   // position of block row m: its sequence's context length + m % 16
  };
  __device__ __forceinline__ Row row(int m) const { return Row{ctx_len[m >> 4] + (m & 15)}; }
  __device__ __forceinline__ bool colmajor(int vt) const { return vt >= (H + Hkv) * hd / 16; }
  // destination of tile vt: kind 0 query, 1 key (both rotated, base at the head; inv = the
  // inverse frequencies of its 8 dimension pairs), 2 value (base at the tile's first
  // dimension), -1 none
  struct Col {
    double inv[8];
    T* p;
    int kind, tt;
  };
  __device__ __forceinline__ Col col(int vt) const {
    const int tq = H * hd / 16, tk = Hkv * hd / 16, tph = hd / 16;
    Col cf{};
    cf.kind = -1;
    if (vt < tq) {
      cf = Col{{}, q + (vt / tph) * hd, 0, vt % tph};
    } else if (vt - tq < tk) {
      cf = Col{{}, kb + ((vt - tq) / tph) * 16 * hd, 1, (vt - tq) % tph};
    } else if (vt - tq - tk < tk) {
      cf = Col{{}, vbt + (vt - tq - tk) * 16 * 16, 2, 0};   // value dims from (vt-tq-tk)*16 (no head straddles a tile)
    }
    if (cf.kind == 0 || cf.kind == 1)
      for (int j = 0; j < 8; ++j) cf.inv[j] = rf.inv[8 * cf.tt + j];
    return cf;
  }
  __device__ __forceinline__ void put(T* p, int kind, int tt, double inv, int m, const Row& rw, int c, float v,
                                      float pv) const {
    const int b = m >> 4, j = m & 15;
    if (kind < 0) return;
    if (kind < 2) {
      const int dim = rope_dim(tt, c, hd);
      float cs, sn;
      rope_cs(rw.pos, inv, &cs, &sn);
      const float r = (c < 8) ? v * cs - pv * sn : v * cs + pv * sn;
      if (kind == 0) p[static_cast<size_t>(m) * H * hd + dim] = from_f<T>(r);
      else p[(static_cast<size_t>(b) * Hkv * 16 + j) * hd + dim] = from_f<T>(r);
    } else {
      p[static_cast<size_t>(b) * Hkv * hd * 16 + c * 16 + j] = from_f<T>(v);
    }
  }
  // cf: facts of the tile held in shared memory (read in place)
  __device__ __forceinline__ void apply(const Col& cf, int m, const Row& rw, int c, float v, float pv) const {
    const int kind = cf.kind;
    put(cf.p, kind, cf.tt, kind == 0 || kind == 1 ? cf.inv[c & 7] : 0.0, m, rw, c, v, pv);
  }
  static constexpr bool kRope = true;
  __device__ __forceinline__ int rope_pairs() const { return hd / 2; }
  __device__ __forceinline__ double rope_inv(int j) const { return rf.inv[j]; }
  __device__ __forceinline__ void apply(const Col& cf, int m, const Row&, int c, float v, float pv,
                                        const float2* cs_row) const {
    const int kind = cf.kind, b = m >> 4, j = m & 15;
    if (kind < 0) return;
    if (kind < 2) {
      const float2 t = cs_row[8 * cf.tt + (c & 7)];
      const float r = (c < 8) ? v * t.x - pv * t.y : v * t.x + pv * t.y;
      const int dim = rope_dim(cf.tt, c, hd);
      if (kind == 0) cf.p[static_cast<size_t>(m) * H * hd + dim] = from_f<T>(r);
      else cf.p[(static_cast<size_t>(b) * Hkv * 16 + j) * hd + dim] = from_f<T>(r);
    } else {
      cf.p[static_cast<size_t>(b) * Hkv * hd * 16 + c * 16 + j] = from_f<T>(v);
    }
  }
  __device__ __forceinline__ int kind8(const Col& cf) const { return cf.kind < 0 ? -1 : (cf.kind < 2 ? 1 : 0); }
  __device__ __forceinline__ void store8_rot(const Col& cf, int m, const Row&, int h, const float (&o)[8]) const {
    const int dim0 = rope_dim(cf.tt, 8 * h, hd), b = m >> 4, j = m & 15;
    if (cf.kind == 0) store8(cf.p + static_cast<size_t>(m) * H * hd + dim0, o);
    else store8(cf.p + (static_cast<size_t>(b) * Hkv * 16 + j) * hd + dim0, o);
  }
  // rows m0 .. m0+7 lie in one 16-row block (m0 % 8 == 0)
  __device__ __forceinline__ void store8_val(const Col& cf, int m0, const Row*, int c, const float (&o)[8],
                                             int M) const {
    T* p = cf.p + static_cast<size_t>(m0 >> 4) * Hkv * hd * 16 + c * 16 + (m0 & 15);
    if (m0 + 8 <= M) {
      store8(p, o);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (m0 + k < M) p[k] = from_f<T>(o[k]);
    }
  }
  __device__ __forceinline__ void apply(int vt, int m, const Row& rw, int c, float v, float pv) const {
    const int tq = H * hd / 16, tk = Hkv * hd / 16, tph = hd / 16;
    if (vt < tq) put(q + (vt / tph) * hd, 0, vt % tph, rf.inv[8 * (vt % tph) + (c & 7)], m, rw, c, v, pv);
    else if (vt - tq < tk)
      put(kb + ((vt - tq) / tph) * 16 * hd, 1, (vt - tq) % tph, rf.inv[8 * ((vt - tq) % tph) + (c & 7)], m, rw, c, v, pv);
    else if (vt - tq - tk < tk) put(vbt + (vt - tq - tk) * 16 * 16, 2, 0, 0.0, m, rw, c, v, pv);
  }
};

// ------------------------------------------------------------------ context K/V injection

template <typename T>
struct EpiInject {
  const T* wk[16];
  const T* wv[16];
  T* kc[16];
  T* vtc[16];
  int K, L, Hkv, hd, B, cap;
  RopeFreq rf;             // inverse rotary frequencies
  const int32_t* row_off;  // [B+1]
  const int32_t* pos0;     // [B]
  const int32_t* n_new;    // [B]
  static constexpr int PX = 0, PC = 8;
  static constexpr bool kDirect = false;
  static constexpr bool kTop16 = false;
  // virtual tiles per layer: Hkv*hd/16 key tiles (RoPE-paired) then Hkv*hd/16 value tiles
  __device__ __forceinline__ const T* wrow(int vt, int c) const {
    const int tk = Hkv * hd / 16, tph = hd / 16;
    const int l = vt / (2 * tk), t = vt % (2 * tk);
    if (l >= L) return nullptr;
    if (t < tk) return wk[l] + static_cast<size_t>((t / tph) * hd + rope_dim(t % tph, c, hd)) * K;
    return wv[l] + static_cast<size_t>((t - tk) * 16 + c) * K;
  }
  __device__ __forceinline__ void wseg(int vt, const T*& b, uint32_t& n) const {
    const int tk = Hkv * hd / 16;
    const int l = vt / (2 * tk), t = vt % (2 * tk);
    if (l >= L) {
      b = wk[0];
      n = 0;
      return;
    }
    b = t < tk ? wk[l] : wv[l];
    n = static_cast<uint32_t>(static_cast<size_t>(Hkv) * hd * K * sizeof(T));
  }
  struct Row {
    int b, pos;   // owning sequence and cache position of row m; b < 0: row not stored
  };
  // sequence owning row m: row_off[b] <= m < row_off[b+1]; rows past n_new[b] or outside
  // the cache are dropped
  __device__ __forceinline__ Row row(int m) const {
    if (m < row_off[0] || m >= row_off[B]) return Row{-1, 0};
    int lo = 0, hi = B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (row_off[mid] <= m) lo = mid; else hi = mid;
    }
    const int i = m - row_off[lo];
    const int pos = pos0[lo] + i;
    if (i >= n_new[lo] || pos < 0 || pos >= cap) return Row{-1, 0};
    return Row{lo, pos};
  }
  __device__ __forceinline__ bool colmajor(int vt) const { return vt % (2 * (Hkv * hd / 16)) >= Hkv * hd / 16; }
  // destination of tile vt: kind 0 key (rotated; base at the head; inv = the inverse
  // frequencies of its 8 dimension pairs), 1 value (base at the tile's first dimension), -1 none
  struct Col {
    double inv[8];
    T* p;
    int kind, tt;
  };
  __device__ __forceinline__ Col col(int vt) const {
    const int tk = Hkv * hd / 16, tph = hd / 16;
    const int l = vt / (2 * tk), t = vt % (2 * tk);
    Col cf{};
    cf.kind = -1;
    if (l >= L) return cf;
    if (t < tk) {
      cf = Col{{}, kc[l] + static_cast<size_t>(t / tph) * cap * hd, 0, t % tph};
      for (int j = 0; j < 8; ++j) cf.inv[j] = rf.inv[8 * cf.tt + j];
    } else {
      cf = Col{{}, vtc[l] + static_cast<size_t>(t - tk) * 16 * cap, 1, 0};   // value dims (t-tk)*16.. of the layer
    }
    return cf;
  }
  __device__ __forceinline__ void put(T* p, int kind, int tt, double inv, const Row& rw, int c, float v,
                                      float pv) const {
    if (kind < 0 || rw.b < 0) return;
    const size_t bo = static_cast<size_t>(rw.b) * Hkv * cap * hd;
    if (kind == 0) {
      float cs, sn;
      rope_cs(rw.pos, inv, &cs, &sn);
      const float r = (c < 8) ? v * cs - pv * sn : v * cs + pv * sn;
      p[bo + static_cast<size_t>(rw.pos) * hd + rope_dim(tt, c, hd)] = from_f<T>(r);
    } else {
      p[bo + static_cast<size_t>(c) * cap + rw.pos] = from_f<T>(v);
    }
  }
  // cf: facts of the tile held in shared memory (read in place)
  __device__ __forceinline__ void apply(const Col& cf, int, const Row& rw, int c, float v, float pv) const {
    const int kind = cf.kind;
    put(cf.p, kind, cf.tt, kind == 0 ? cf.inv[c & 7] : 0.0, rw, c, v, pv);
  }
  static constexpr bool kRope = true;
  __device__ __forceinline__ int rope_pairs() const { return hd / 2; }
  __device__ __forceinline__ double rope_inv(int j) const { return rf.inv[j]; }
  __device__ __forceinline__ void apply(const Col& cf, int, const Row& rw, int c, float v, float pv,
                                        const float2* cs_row) const {
    const int kind = cf.kind;
    if (kind < 0 || rw.b < 0) return;
    const size_t bo = static_cast<size_t>(rw.b) * Hkv * cap * hd;
    if (kind == 0) {
      const float2 t = cs_row[8 * cf.tt + (c & 7)];
      const float r = (c < 8) ? v * t.x - pv * t.y : v * t.x + pv * t.y;
      cf.p[bo + static_cast<size_t>(rw.pos) * hd + rope_dim(cf.tt, c, hd)] = from_f<T>(r);
    } else {
      cf.p[bo + static_cast<size_t>(c) * cap + rw.pos] = from_f<T>(v);
    }
  }
  __device__ __forceinline__ int kind8(const Col& cf) const { return cf.kind < 0 ? -1 : (cf.kind == 0 ? 1 : 0); }
  __device__ __forceinline__ void store8_rot(const Col& cf, int, const Row& rw, int h, const float (&o)[8]) const {
    if (rw.b < 0) return;
    store8(cf.p + static_cast<size_t>(rw.b) * Hkv * cap * hd + static_cast<size_t>(rw.pos) * hd +
               rope_dim(cf.tt, 8 * h, hd), o);
  }
  // column c of rows m0 .. m0+7: one 8-wide store when they are 8 consecutive cache positions of
  // one sequence, else row by row (rows not stored skipped)
  __device__ __forceinline__ void store8_val(const Col& cf, int m0, const Row* rows, int c, const float (&o)[8],
                                             int M) const {
    const Row r0 = rows[0], r7 = rows[7];
    if (m0 + 8 <= M && r0.b >= 0 && r7.b == r0.b && r7.pos == r0.pos + 7) {
      store8(cf.p + static_cast<size_t>(r0.b) * Hkv * cap * hd + static_cast<size_t>(c) * cap + r0.pos, o);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const Row rk = rows[k];
        if (m0 + k < M && rk.b >= 0)
          cf.p[static_cast<size_t>(rk.b) * Hkv * cap * hd + static_cast<size_t>(c) * cap + rk.pos] = from_f<T>(o[k]);
      }
    }
  }
  __device__ __forceinline__ void apply(int vt, int, const Row& rw, int c, float v, float pv) const {
    const int tk = Hkv * hd / 16, tph = hd / 16;
    const int l = vt / (2 * tk), t = vt % (2 * tk);
    if (l >= L) return;
    if (t < tk) put(kc[l] + static_cast<size_t>(t / tph) * cap * hd, 0, t % tph, rf.inv[8 * (t % tph) + (c & 7)], rw, c, v, pv);
    else put(vtc[l] + static_cast<size_t>(t - tk) * 16 * cap, 1, 0, 0.0, rw, c, v, pv);
  }
};

// ------------------------------------------------------------------ SwiGLU (gate/up pair)

template <typename T>
struct EpiSwiGLU {
  const T* wg;
  const T* wu;
  int K, Fd;
  T* h;  // [M][Fd]
  static constexpr int PX = 1, PC = 0;
  static constexpr bool kDirect = true;
  static constexpr bool kTop16 = false;
  __device__ __forceinline__ const T* wrow(int vt, int c) const {
    const int n = (vt >> 1) * 16 + c;
    if (n >= Fd) return nullptr;
    return ((vt & 1) ? wu : wg) + static_cast<size_t>(n) * K;
  }
  __device__ __forceinline__ void wseg(int vt, const T*& b, uint32_t& n) const {
    b = (vt & 1) ? wu : wg;
    n = (vt >> 1) * 16 < Fd ? static_cast<uint32_t>(static_cast<size_t>(Fd) * K * sizeof(T)) : 0u;
  }
  struct Row {};
  __device__ __forceinline__ Row row(int) const { return Row{}; }
  __device__ __forceinline__ bool colmajor(int) const { return false; }
  __device__ __forceinline__ void apply(int vt, int m, const Row&, int c, float v, float pv) const {
    if (vt & 1) return;
    const int n = (vt >> 1) * 16 + c;
    if (n >= Fd) return;
    const float s = v / (1.f + expf(-v));
    h[static_cast<size_t>(m) * Fd + n] = from_f<T>(s * pv);
  }
  // four consecutive outputs n..n+3 of row m from their gate and up sums (the staged
  // epilogues): one 8-byte store where the row allows it, the same values as apply()
  static constexpr bool kPair4 = true;
  __device__ __forceinline__ void apply_pair4(int m, int n, const float* g, const float* u) const {
    float o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = g[k] / (1.f + expf(-g[k])) * u[k];
    T* p = h + static_cast<size_t>(m) * Fd + n;
    if (sizeof(T) == 2 && n + 4 <= Fd && (reinterpret_cast<uintptr_t>(p) & 7) == 0) {
      const uint2 w = {static_cast<uint32_t>(from_f<T>(o[0])) | (static_cast<uint32_t>(from_f<T>(o[1])) << 16),
                       static_cast<uint32_t>(from_f<T>(o[2])) | (static_cast<uint32_t>(from_f<T>(o[3])) << 16)};
      *reinterpret_cast<uint2*>(p) = w;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (n + k < Fd) p[k] = from_f<T>(o[k]);
    }
  }
};

}  // namespace dflash
