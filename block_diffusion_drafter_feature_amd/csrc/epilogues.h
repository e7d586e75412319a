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
#pragma once

#include "common.h"

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
};

// LM-head logits: a plain fp32 store, kept as its own type so that the LM-head GEMM is a
// kernel of its own in profiles.  With tmax != nullptr the pipelined kernel (unsplit, 128-
// column tiles) also writes each row's maximum over every 128-column group of the logits,
// tmax[m][n / 128] (columns past the vocabulary excluded).
template <typename T>
struct EpiLogits : EpiStore<T> {
  float* tmax;
};
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
  __device__ __forceinline__ void apply(int vt, int m, const Row& rw, int c, float v, float pv) const {
    const int tq = H * hd / 16, tk = Hkv * hd / 16, tph = hd / 16;
    const int b = m >> 4, j = m & 15;
    if (vt < tq + tk) {
      const bool isq = vt < tq;
      const int t = isq ? vt : vt - tq;
      const int head = t / tph, tt = t % tph;
      const int dim = rope_dim(tt, c, hd);
      float cs, sn;
      rope_cs(rw.pos, rf.inv[8 * tt + (c & 7)], &cs, &sn);
      const float r = (c < 8) ? v * cs - pv * sn : v * cs + pv * sn;
      if (isq) q[(static_cast<size_t>(m) * H + head) * hd + dim] = from_f<T>(r);
      else kb[((static_cast<size_t>(b) * Hkv + head) * 16 + j) * hd + dim] = from_f<T>(r);
    } else {
      const int t = vt - tq - tk;
      if (t >= tk) return;
      const int n = t * 16 + c, head = n / hd, dim = n % hd;
      vbt[((static_cast<size_t>(b) * Hkv + head) * hd + dim) * 16 + j] = from_f<T>(v);
    }
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
  __device__ __forceinline__ void apply(int vt, int m, const Row& rw, int c, float v, float pv) const {
    const int tk = Hkv * hd / 16, tph = hd / 16;
    const int l = vt / (2 * tk), t = vt % (2 * tk);
    if (l >= L || rw.b < 0) return;
    const int b = rw.b, pos = rw.pos;
    if (t < tk) {
      const int head = t / tph, tt = t % tph, dim = rope_dim(tt, c, hd);
      float cs, sn;
      rope_cs(pos, rf.inv[8 * tt + (c & 7)], &cs, &sn);
      const float r = (c < 8) ? v * cs - pv * sn : v * cs + pv * sn;
      kc[l][((static_cast<size_t>(b) * Hkv + head) * cap + pos) * hd + dim] = from_f<T>(r);
    } else {
      const int n = (t - tk) * 16 + c, head = n / hd, dim = n % hd;
      vtc[l][((static_cast<size_t>(b) * Hkv + head) * hd + dim) * cap + pos] = from_f<T>(v);
    }
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
};

}  // namespace dflash
