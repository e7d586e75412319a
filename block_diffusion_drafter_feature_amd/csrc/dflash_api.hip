// C ABI of the drafting step: argument checks, workspace carving and the launch
// sequence of each call.  Every call validates all of its arguments before the
// first launch, then enqueues its kernels on the caller's stream and returns.
#include "dflash.h"

#include "attention.h"
#include <cmath>
#include "common.h"
#include "conv.h"
#include "elementwise.h"
#include "epilogues.h"
#include "gemm.h"
#include "select.h"

#include <algorithm>
#include <atomic>

using namespace dflash;

namespace {

constexpr size_t kAlign = 256;
constexpr int kTopkChunk = kTopkWaveChunk;   // vocabulary columns per top-k wave
constexpr int kTopkTilesNG = 20;              // 128-column groups per lane in topk_tiles_kernel
constexpr int kArgmaxChunk = 8192;   // vocabulary columns per argmax work-group
constexpr int kTopkFinalLists = 256;  // lists topk_final_kernel merges per row (64 lanes x 4)

size_t align_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

// Carves typed slices out of the caller's workspace; with base == nullptr it only
// adds up the sizes (the *_workspace_bytes queries use the same code).
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename X>
  X* take(size_t n) {
    X* p = base ? reinterpret_cast<X*>(base + off) : nullptr;
    off += align_up(n * sizeof(X));
    return p;
  }
};

size_t esize(const dflash_config* c) { return c->dtype == DFLASH_BF16 ? 2 : 4; }

int check_config(const dflash_config* c) {
  if (!c) return DFLASH_E_INVAL;
  if (c->dtype != DFLASH_BF16 && c->dtype != DFLASH_F32) return DFLASH_E_INVAL;
  if (c->d_model <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 || c->d_ffn <= 0 ||
      c->n_layers <= 0 || c->n_feat_layers <= 0 || c->d_target <= 0 || c->vocab <= 0 || c->ps_dim <= 0 ||
      c->ps_rank <= 0)
    return DFLASH_E_INVAL;
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f) || (c->use_conv != 0 && c->use_conv != 1) ||
      (c->use_gate != 0 && c->use_gate != 1))
    return DFLASH_E_INVAL;
  if (c->n_layers > DFLASH_MAX_LAYERS) return DFLASH_E_UNSUPPORTED;
  if (c->d_model % 64 || c->d_ffn % 64) return DFLASH_E_UNSUPPORTED;
  if (static_cast<int64_t>(c->n_feat_layers) * c->d_target % 64) return DFLASH_E_UNSUPPORTED;
  if (static_cast<int64_t>(c->n_feat_layers) * c->d_target > (1 << 28)) return DFLASH_E_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return DFLASH_E_UNSUPPORTED;
  if (c->n_heads % c->n_kv_heads) return DFLASH_E_UNSUPPORTED;
  const int G = c->n_heads / c->n_kv_heads;
  if (G != 1 && G != 2 && G != 4) return DFLASH_E_UNSUPPORTED;
  if (c->vocab % 16 || c->vocab < 16) return DFLASH_E_UNSUPPORTED;
  if (c->vocab > 256 * kTopkChunk) return DFLASH_E_UNSUPPORTED;     // top-k merges <= 256 chunk lists
  if (c->ps_dim % 64 || c->ps_rank > 256) return DFLASH_E_UNSUPPORTED;
  if (c->weight_format != DFLASH_WEIGHTS_DTYPE && c->weight_format != DFLASH_WEIGHTS_FP8) return DFLASH_E_INVAL;
  if (c->weight_format == DFLASH_WEIGHTS_FP8 && c->dtype != DFLASH_BF16) return DFLASH_E_UNSUPPORTED;
  if (c->block_size < 1 || c->block_size > DFLASH_BLOCK) return DFLASH_E_INVAL;
  if (c->cal_dim < 0 || c->cal_dim % 64) return DFLASH_E_INVAL;
  return DFLASH_OK;
}

int check_weights(const dflash_config* c, const dflash_weights* w, bool draft, bool inject, bool path) {
  if (!w) return DFLASH_E_INVAL;
  if (draft && (!w->embed || !w->lm_head || !w->g_final)) return DFLASH_E_INVAL;
  if (inject && (!w->w_fc || !w->g_fc)) return DFLASH_E_INVAL;
  if (path && (!w->embed || !w->ps_left || !w->ps_right || !w->ps_u || !w->ps_v)) return DFLASH_E_INVAL;
  if (path && c->use_gate && !w->ps_gate) return DFLASH_E_INVAL;
  for (int l = 0; l < c->n_layers; ++l) {
    const dflash_layer_weights& L = w->layers[l];
    if ((draft || inject) && (!L.w_k || !L.w_v)) return DFLASH_E_INVAL;
    if (draft && (!L.w_q || !L.w_o || !L.w_gate || !L.w_up || !L.w_down || !L.g_attn || !L.g_ffn))
      return DFLASH_E_INVAL;
    if (draft && c->use_conv)
      for (int s = 0; s < DFLASH_CONV_SITES; ++s)
        if (!L.conv_gen[s] || !L.conv_w0[s] || !L.conv_w1[s]) return DFLASH_E_INVAL;
  }
  return DFLASH_OK;
}

// The attention kernel addresses one (sequence, kv head) slice of the cache through a
// buffer descriptor with 32-bit offsets and takes 2^31 as its "past the end" offset, so a
// slice (cap rows of head_dim elements) must stay below 2 GiB.
bool kv_slice_ok(const dflash_config* c, int cap) {
  return static_cast<int64_t>(cap) * c->head_dim * static_cast<int64_t>(esize(c)) < (int64_t{1} << 31);
}

int check_kv(const dflash_config* c, const dflash_kv* kv, int batch) {
  if (!kv || kv->cap <= 0 || kv->batch <= 0) return DFLASH_E_INVAL;
  if (kv->cap % 32 || !kv_slice_ok(c, kv->cap)) return DFLASH_E_UNSUPPORTED;
  if (batch > kv->batch) return DFLASH_E_CAPACITY;
  for (int l = 0; l < c->n_layers; ++l)
    if (!kv->k[l] || !kv->vt[l]) return DFLASH_E_INVAL;
  return DFLASH_OK;
}

// ------------------------------------------------------------------ workspace layouts

template <typename T>
struct InjectWs {
  float* hf;   // [rows][d] fused feature before its norm
  T* f;        // [rows][d] fused feature, storage type
  float* scratch;
  size_t scratch_bytes;
};
template <typename T>
InjectWs<T> carve_inject(Carver& cv, const dflash_config* c, int rows) {
  InjectWs<T> w;
  const int d = c->d_model, dcat = c->n_feat_layers * c->d_target;
  w.hf = cv.take<float>(static_cast<size_t>(rows) * d);
  w.f = cv.take<T>(static_cast<size_t>(rows) * d);
  w.scratch_bytes = std::max(splitk_scratch_bytes<T>(rows, dcat, (d + 15) / 16),
                             splitk_scratch_bytes<T>(rows, d, c->n_layers * 2 * c->n_kv_heads * c->head_dim / 16));
  w.scratch = cv.take<float>(w.scratch_bytes / sizeof(float) + 1);
  return w;
}

// Context splits per (sequence, kv head): about two four-wave work-groups per compute
// unit over the grid, each split at least four 64-key tiles of a full cache (so the 32 KB
// of (O, m, l) partials a split writes stay well below the K/V bytes it reads; at batch 1,
// context 4096, 16 or 32 splits take 23 us per layer against 25.6 us for 64), at most 64.
int attn_splits(const dflash_config* c, int batch, int cap) {
  // about 512 work-groups (two per CU), and at least 4 splits: with many sequences the
  // longest contexts otherwise set the time (32 x 4096 keys: 2 splits 165 us, 4 splits 143 us)
  // With 256+ (sequence, kv head) pairs, splits of at most ~1024 keys: every sequence is cut
  // by the batch's longest context, so in a ragged batch the long contexts spread over more
  // work-groups while short ones leave splits empty (they exit at once).
  const int pairs = batch * c->n_kv_heads;
  int want = std::max((512 + pairs - 1) / pairs, 4);
  if (pairs >= 256) want = std::max(want, std::min(cap / 1024, 16));
  const int maxs = cap / 256;
  int s = want < maxs ? want : maxs;
  s = s < 1 ? 1 : (s > kCombineMaxSplits ? kCombineMaxSplits : s);
  // a small grid (latency-bound: batch 1) gives the block's own keys a split of their own
  if (s > 1 && s < kCombineMaxSplits && pairs * (s + 1) <= 256) ++s;
  return s;
}

// Context splits of a launch with S splits (see attn_splits): S - 1 when the last split
// holds only the block keys.
int attn_ctx_splits(const dflash_config* c, int batch, int cap, int S) {
  return S > 1 && batch * c->n_kv_heads * S <= 256 ? S - 1 : S;
}

template <typename T>
struct DraftWs {
  float* x;       // [M][d] residual stream
  float* uf;      // [M][d] sublayer GEMM output before the conv, fp32
  float* ss;      // [M][d/256 rounded up] partial sums of squares of x rows (conv kernels)
  T* ut;          // [M][d] GEMM operand
  T* q;           // [M][H*hd]
  T* kb;          // [B][Hkv][16][hd]
  T* vbt;         // [B][Hkv][hd][16]
  float* part_o;  // [B][Hkv][S][G][16][hd]
  float* part_ml;
  T* o;           // [M][H*hd]
  T* h;           // [M][d_ffn]
  float* logits;  // [M][V] (when the caller passes none)
  float* tmax;    // [M][V/128 rounded up] row maxima of the logits per 128-column group
  float* tk_v;    // [M][n_chunks][16]
  int32_t* tk_i;
  float* scratch;
  size_t scratch_bytes;
  int S, SC;
};
template <typename T>
DraftWs<T> carve_draft(Carver& cv, const dflash_config* c, int B, int cap) {
  DraftWs<T> w;
  const size_t M = 16 * static_cast<size_t>(B), d = c->d_model, hq = static_cast<size_t>(c->n_heads) * c->head_dim;
  const int G = c->n_heads / c->n_kv_heads;
  w.S = attn_splits(c, B, cap);
  w.SC = attn_ctx_splits(c, B, cap, w.S);
  const int nch = (c->vocab + kTopkChunk - 1) / kTopkChunk;
  w.x = cv.take<float>(M * d);
  w.uf = cv.take<float>(M * d);
  w.ss = cv.take<float>(M * ((d / 16 + 15) / 16));
  w.ut = cv.take<T>(M * d);
  w.q = cv.take<T>(M * hq);
  w.kb = cv.take<T>(static_cast<size_t>(B) * c->n_kv_heads * 16 * c->head_dim);
  w.vbt = cv.take<T>(static_cast<size_t>(B) * c->n_kv_heads * 16 * c->head_dim);
  w.part_o = cv.take<float>(static_cast<size_t>(B) * c->n_kv_heads * w.S * G * 16 * c->head_dim);
  w.part_ml = cv.take<float>(static_cast<size_t>(B) * c->n_kv_heads * w.S * G * 16 * 2);
  w.o = cv.take<T>(M * hq);
  w.h = cv.take<T>(M * c->d_ffn);
  w.logits = cv.take<float>(M * c->vocab);
  w.tmax = cv.take<float>(M * ((c->vocab + 127) / 128));
  // top-16 partial lists: one per vocabulary chunk, or one per LM-head work-group when
  // the first stage runs in the streaming LM head (at most kTopkFinalLists)
  const size_t ntk = std::max<size_t>(nch, kTopkFinalLists);
  w.tk_v = cv.take<float>(M * ntk * 16);
  w.tk_i = cv.take<int32_t>(M * ntk * 16);
  const int Mi = static_cast<int>(M), di = c->d_model, hqi = c->n_heads * c->head_dim;
  const int hki = c->n_kv_heads * c->head_dim, F = c->d_ffn;
  size_t sc = 0;
  sc = std::max(sc, splitk_scratch_bytes<T>(Mi, di, (hqi + 2 * hki) / 16));
  sc = std::max(sc, splitk_scratch_bytes<T>(Mi, hqi, di / 16));
  sc = std::max(sc, splitk_scratch_bytes<T>(Mi, di, 2 * (F / 16)));
  sc = std::max(sc, splitk_scratch_bytes<T>(Mi, F, di / 16));
  sc = std::max(sc, splitk_scratch_bytes<T>(Mi, di, c->vocab / 16));
  w.scratch_bytes = sc;
  w.scratch = cv.take<float>(sc / sizeof(float) + 1);
  return w;
}

constexpr int kPathSlots = 16 * 16 + 1;

struct PathWs {
  int32_t* tokens;  // [B][T]
  float* z;         // [B][T][2*PD]
  float* gamma;     // [B*16][PD]
  float* S;         // [B][16][16][16] pair scores
  void* xb;         // [B*16][d] final hidden rounded to the weights' type (bf16 only)
  float* scratch;
  size_t scratch_bytes;
};
template <typename X>
PathWs carve_path(Carver& cv, const dflash_config* c, int B) {
  PathWs w;
  const size_t T = kPathSlots;
  w.tokens = cv.take<int32_t>(B * T);
  w.z = cv.take<float>(B * T * 2 * c->ps_dim);
  w.gamma = cv.take<float>(static_cast<size_t>(B) * 16 * c->ps_dim);
  w.S = cv.take<float>(static_cast<size_t>(B) * 16 * 256);
  w.xb = std::is_same<X, bf16_t>::value ? cv.take<X>(static_cast<size_t>(B) * 16 * c->d_model) : nullptr;
  size_t sc = 0;
  for (int nf = 0; nf < 2; ++nf)
    sc = std::max(sc, splitk_scratch_bytes<X>(B * (16 * (16 - nf) + nf), c->d_model, 2 * c->ps_dim / 16));
  sc = std::max(sc, splitk_scratch_bytes<X>(16 * B, c->d_model, c->ps_dim / 16));
  w.scratch_bytes = sc;
  w.scratch = cv.take<float>(sc / sizeof(float) + 1);
  return w;
}

struct VerifyWs {
  float* pv;
  int32_t* pi;
};
VerifyWs carve_verify(Carver& cv, int B, int n_draft, int V) {
  VerifyWs w;
  const size_t nch = (V + kArgmaxChunk - 1) / kArgmaxChunk;
  w.pv = cv.take<float>(static_cast<size_t>(B) * (n_draft + 1) * nch);
  w.pi = cv.take<int32_t>(static_cast<size_t>(B) * (n_draft + 1) * nch);
  return w;
}

template <typename T>
struct CalWs {
  T* a;          // [M][2d] MLP input
  float* h;      // [M][cal_dim] hidden layer
  float* tk_v;   // [M][n_chunks][16]
  int32_t* tk_i;
  float* scratch;
  size_t scratch_bytes;
};
template <typename T>
CalWs<T> carve_cal(Carver& cv, const dflash_config* c, int B) {
  CalWs<T> w;
  const size_t M = static_cast<size_t>(16) * B, d = c->d_model, nch = (c->vocab + kTopkChunk - 1) / kTopkChunk;
  w.a = cv.take<T>(M * 2 * d);
  w.h = cv.take<float>(M * c->cal_dim);
  w.tk_v = cv.take<float>(M * nch * 16);
  w.tk_i = cv.take<int32_t>(M * nch * 16);
  w.scratch_bytes = std::max(splitk_scratch_bytes<T>(static_cast<int>(M), 2 * c->d_model, c->cal_dim / 16),
                             splitk_scratch_bytes<T>(static_cast<int>(M), c->cal_dim, c->vocab / 16));
  w.scratch = cv.take<float>(w.scratch_bytes / sizeof(float) + 1);
  return w;
}

struct VerifySampledWs {
  float* pm;
  float* ps;
  BonusSel* sel;
};
VerifySampledWs carve_verify_sampled(Carver& cv, int B, int n_draft, int V) {
  VerifySampledWs w;
  const size_t nch = (V + kSoftmaxChunk - 1) / kSoftmaxChunk;
  w.pm = cv.take<float>(static_cast<size_t>(B) * (n_draft + 1) * nch);
  w.ps = cv.take<float>(static_cast<size_t>(B) * (n_draft + 1) * nch);
  w.sel = cv.take<BonusSel>(static_cast<size_t>(B));
  return w;
}

// log2(e) / t, the exponent scale of a softmax at temperature t; 0 for an invalid t
float temp_scale(float t) {
  if (!(t > 0.f) || !std::isfinite(t)) return 0.f;
  const double k = 1.4426950408889634 / static_cast<double>(t);
  return std::isfinite(static_cast<float>(k)) ? static_cast<float>(k) : 0.f;
}

struct Probe {
  const dflash_probes* p;
  hipStream_t s;
  void begin(int i) const {
    if (p && p->begin[i]) (void)hipEventRecord(p->begin[i], s);
  }
  void end(int i) const {
    if (p && p->end[i]) (void)hipEventRecord(p->end[i], s);
  }
};

#define LAUNCH_CHECK()                             \
  do {                                             \
    if (hipGetLastError() != hipSuccess) return DFLASH_E_HIP; \
  } while (0)
#define GEMM_CHECK(expr)                                      \
  do {                                                        \
    const hipError_t e_ = (expr);                             \
    if (e_ == hipErrorNotSupported) return DFLASH_E_UNSUPPORTED; \
    if (e_ != hipSuccess) return DFLASH_E_HIP;                \
  } while (0)

// FP8 storage of the streamed projections: W rows are K codes + 16 bytes, so the row
// stride the epilogues step by (in T elements) is (K + 16) / 2.
bool fp8w(const dflash_config* c) { return c->weight_format == DFLASH_WEIGHTS_FP8; }
int wstride(const dflash_config* c, int K) { return fp8w(c) ? (K + 16) / 2 : K; }

template <typename T>
SegW<T> seg1(const void* p, int rows, int K) {
  SegW<T> s{};
  s.p[0] = static_cast<const T*>(p);
  s.off[0] = 0;
  s.off[1] = rows;
  s.n_seg = 1;
  s.K = K;
  return s;
}

// ------------------------------------------------------------------ inject

template <typename T>
int inject_impl(const dflash_config* c, const dflash_weights* w, const dflash_kv* kv, const void* hidden,
                int rows, const int32_t* row_off, const int32_t* pos0, const int32_t* n_new, int B, void* ws,
                const Probe& pr, hipStream_t s) {
  Carver cv(ws);
  InjectWs<T> W = carve_inject<T>(cv, c, rows);
  const int d = c->d_model, dcat = c->n_feat_layers * c->d_target;
  {
    EpiStore<T> e{seg1<T>(w->w_fc, d, wstride(c, dcat)), W.hf, d, STORE};
    pr.begin(DFLASH_PROBE_INJECT_FC);
    GEMM_CHECK((run_gemm<T, T>(static_cast<const T*>(hidden), dcat, nullptr, rows, dcat, (d + 15) / 16, e, s,
                               W.scratch, W.scratch_bytes, 0, fp8w(c))));
    pr.end(DFLASH_PROBE_INJECT_FC);
  }
  launch_rmsnorm<T>(rows, s, W.hf, static_cast<const T*>(w->g_fc), d, c->rms_eps, W.f, nullptr);
  LAUNCH_CHECK();
  EpiInject<T> e{};
  for (int l = 0; l < c->n_layers; ++l) {
    e.wk[l] = static_cast<const T*>(w->layers[l].w_k);
    e.wv[l] = static_cast<const T*>(w->layers[l].w_v);
    e.kc[l] = static_cast<T*>(kv->k[l]);
    e.vtc[l] = static_cast<T*>(kv->vt[l]);
  }
  e.K = wstride(c, d);
  e.L = c->n_layers;
  e.Hkv = c->n_kv_heads;
  e.hd = c->head_dim;
  e.B = B;
  e.cap = kv->cap;
  e.rf = rope_freq(c->rope_theta, c->head_dim);
  e.row_off = row_off;
  e.pos0 = pos0;
  e.n_new = n_new;
  const int nvt = c->n_layers * 2 * c->n_kv_heads * c->head_dim / 16;
  pr.begin(DFLASH_PROBE_INJECT_KV);
  GEMM_CHECK((run_gemm<T, T>(W.f, d, nullptr, rows, d, nvt, e, s, W.scratch, W.scratch_bytes, 0, fp8w(c))));
  pr.end(DFLASH_PROBE_INJECT_KV);
  return DFLASH_OK;
}

// ------------------------------------------------------------------ draft

template <typename T, int HD, int G>
hipError_t launch_attn(const AttnArgs<T>& a, int B, hipStream_t s) {
  dim3 grid(a.S, a.Hkv, B);
  block_attn_kernel<T, HD, G><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

// split partials merge: 2 split groups for S <= 3, else 4; each wave loads NS splits
template <typename T, int HD, int SG, int NS>
hipError_t combine_grid(const AttnArgs<T>& a, int H, int Hkv, int B, hipStream_t s) {
  constexpr int rows_per_block = (64 / (HD / 8)) * (4 / SG);
  attn_combine_kernel<T, HD, SG, NS><<<dim3(16 / rows_per_block, H, B), 256, 0, s>>>(
      a.part_o, a.part_ml, a.out, H, Hkv, a.S, a.ctx_len, B, a.cap, AttnTile<T, HD>::TK, a.SC);
  return hipGetLastError();
}
template <typename T, int HD>
hipError_t launch_combine(const AttnArgs<T>& a, int H, int Hkv, int B, hipStream_t s) {
  const int S = a.S;
  if (S <= 2) return combine_grid<T, HD, 2, 1>(a, H, Hkv, B, s);
  if (S <= 3) return combine_grid<T, HD, 2, 2>(a, H, Hkv, B, s);
  if (S <= 4) return combine_grid<T, HD, 4, 1>(a, H, Hkv, B, s);
  if (S <= 8) return combine_grid<T, HD, 4, 2>(a, H, Hkv, B, s);
  if (S <= 16) return combine_grid<T, HD, 4, 4>(a, H, Hkv, B, s);
  if (S <= 32) return combine_grid<T, HD, 4, 8>(a, H, Hkv, B, s);
  return combine_grid<T, HD, 4, 16>(a, H, Hkv, B, s);
}

template <typename T>
hipError_t run_attention(const dflash_config* c, const AttnArgs<T>& a, int B, hipStream_t s) {
  const int G = c->n_heads / c->n_kv_heads;
  hipError_t e;
  if (c->head_dim == 64) {
    e = G == 1 ? launch_attn<T, 64, 1>(a, B, s) : G == 2 ? launch_attn<T, 64, 2>(a, B, s) : launch_attn<T, 64, 4>(a, B, s);
  } else {
    e = G == 1 ? launch_attn<T, 128, 1>(a, B, s) : G == 2 ? launch_attn<T, 128, 2>(a, B, s) : launch_attn<T, 128, 4>(a, B, s);
  }
  if (e != hipSuccess || a.S == 1) return e;
  return c->head_dim == 64 ? launch_combine<T, 64>(a, c->n_heads, c->n_kv_heads, B, s)
                           : launch_combine<T, 128>(a, c->n_heads, c->n_kv_heads, B, s);
}

// pre-sublayer input: u = RMSNorm(x; g), conv'd when enabled, rounded to T into W.ut (the
// first layer gathers the block's embedding rows into x in the same launch)
template <typename T>
int pre_sublayer(const dflash_config* c, const dflash_layer_weights& L, int site, const void* gain, int M,
                 DraftWs<T>& W, hipStream_t s, const T* emb = nullptr, const int32_t* ids = nullptr,
                 const Probe* pr = nullptr) {
  const int d = c->d_model;
  if (!c->use_conv) {
    launch_rmsnorm<T>(M, s, W.x, static_cast<const T*>(gain), d, c->rms_eps, W.ut, nullptr, emb, ids);
    LAUNCH_CHECK();
    return DFLASH_OK;
  }
  if (pr) pr->begin(DFLASH_PROBE_CONV_PRE);
  // row scales: the first layer's gathered rows are summed in the kernel; later inputs come
  // from a post-sublayer conv, which leaves partial sums of squares of the rows it wrote
  const int tiles = (d / 16 + 15) / 16;
  conv_site_kernel<T, true><<<dim3(tiles, M / 16), 64 * kConvWaves, 0, s>>>(
      W.x, emb, ids, emb ? nullptr : W.ss, tiles, static_cast<const T*>(gain), c->rms_eps,
      static_cast<const T*>(L.conv_gen[site]), static_cast<const T*>(L.conv_w0[site]),
      static_cast<const T*>(L.conv_w1[site]), d, W.x, nullptr, W.ut);
  LAUNCH_CHECK();
  if (pr) pr->end(DFLASH_PROBE_CONV_PRE);
  return DFLASH_OK;
}

// post-sublayer: x += A W^T, through the conv when enabled (the GEMM stores its rows, the
// conv kernel adds the conv'd rows to x)
template <typename T, typename AS>
int post_sublayer(const dflash_config* c, const dflash_layer_weights& L, int site, const void* wmat, const AS* A,
                  int K, int M, DraftWs<T>& W, const Probe& pr, int probe, hipStream_t s) {
  const int d = c->d_model;
  EpiStore<T> e{seg1<T>(wmat, d, wstride(c, K)), c->use_conv ? W.uf : W.x, d, c->use_conv ? STORE : ADD};
  pr.begin(probe);
  GEMM_CHECK((run_gemm<T, AS>(A, K, nullptr, M, K, d / 16, e, s, W.scratch, W.scratch_bytes, 0, fp8w(c))));
  pr.end(probe);
  if (!c->use_conv) return DFLASH_OK;
  if (probe == DFLASH_PROBE_O) pr.begin(DFLASH_PROBE_CONV_POST);
  conv_site_kernel<T, false><<<dim3((d / 16 + 15) / 16, M / 16), 64 * kConvWaves, 0, s>>>(
      W.uf, nullptr, nullptr, nullptr, 0, nullptr, 0.f, static_cast<const T*>(L.conv_gen[site]),
      static_cast<const T*>(L.conv_w0[site]), static_cast<const T*>(L.conv_w1[site]), d, W.x, W.ss, nullptr);
  LAUNCH_CHECK();
  if (probe == DFLASH_PROBE_O) pr.end(DFLASH_PROBE_CONV_POST);
  return DFLASH_OK;
}

template <typename T>
int draft_impl(const dflash_config* c, const dflash_weights* w, const dflash_kv* kv, const int32_t* ctx_len,
               const int32_t* block_ids, int B, int32_t* cand_ids, float* cand_logits, float* final_hidden,
               float* logits, void* ws, const dflash_probes* probes, hipStream_t s) {
  const Probe P0{probes, s}, PN{nullptr, s};
  Carver cv(ws);
  DraftWs<T> W = carve_draft<T>(cv, c, B, kv->cap);
  const int M = 16 * B, d = c->d_model, H = c->n_heads, Hkv = c->n_kv_heads, hd = c->head_dim;
  const int hq = H * hd, F = c->d_ffn, V = c->vocab;
  int rc;
  for (int l = 0; l < c->n_layers; ++l) {
    const dflash_layer_weights& L = w->layers[l];
    const Probe& pr = l == 0 ? P0 : PN;
    // attention sublayer (layer 0: the block's embedding rows are gathered by the same pass)
    if ((rc = pre_sublayer<T>(c, L, 0, L.g_attn, M, W, s, l == 0 ? static_cast<const T*>(w->embed) : nullptr,
                              l == 0 ? block_ids : nullptr)))
      return rc;
    EpiQKV<T> eq{static_cast<const T*>(L.w_q), static_cast<const T*>(L.w_k), static_cast<const T*>(L.w_v),
                 wstride(c, d), H, Hkv, hd, rope_freq(c->rope_theta, hd), ctx_len, W.q, W.kb, W.vbt};
    pr.begin(DFLASH_PROBE_QKV);
    GEMM_CHECK((run_gemm<T, T>(W.ut, d, nullptr, M, d, (hq + 2 * Hkv * hd) / 16, eq, s, W.scratch,
                               W.scratch_bytes, 0, fp8w(c))));
    pr.end(DFLASH_PROBE_QKV);
    AttnArgs<T> aa{W.q, W.kb, W.vbt, static_cast<const T*>(kv->k[l]), static_cast<const T*>(kv->vt[l]), ctx_len,
                   W.part_o, W.part_ml, W.o, H, Hkv, kv->cap, W.S, B, c->block_size,
                   1.4426950408889634f / sqrtf(static_cast<float>(hd))};
    aa.SC = W.SC;
    pr.begin(DFLASH_PROBE_ATTN);
    GEMM_CHECK(run_attention<T>(c, aa, B, s));
    pr.end(DFLASH_PROBE_ATTN);
    if ((rc = post_sublayer<T, T>(c, L, 1, L.w_o, W.o, hq, M, W, pr, DFLASH_PROBE_O, s))) return rc;
    // feed-forward sublayer
    if ((rc = pre_sublayer<T>(c, L, 2, L.g_ffn, M, W, s, nullptr, nullptr, &pr))) return rc;
    EpiSwiGLU<T> ef{static_cast<const T*>(L.w_gate), static_cast<const T*>(L.w_up), wstride(c, d), F, W.h};
    pr.begin(DFLASH_PROBE_GATE_UP);
    GEMM_CHECK((run_gemm<T, T>(W.ut, d, nullptr, M, d, 2 * (F / 16), ef, s, W.scratch, W.scratch_bytes, 0,
                               fp8w(c))));
    pr.end(DFLASH_PROBE_GATE_UP);
    if ((rc = post_sublayer<T, T>(c, L, 3, L.w_down, W.h, F, M, W, pr, DFLASH_PROBE_DOWN, s))) return rc;
  }
  launch_rmsnorm<T>(M, s, W.x, static_cast<const T*>(w->g_final), d, c->rms_eps, W.ut, final_hidden);
  LAUNCH_CHECK();
  float* lg = logits ? logits : W.logits;
  // one drafted block (bf16 or FP8 weights): the streaming LM head keeps each work-group's
  // top 16 per row (the logits are written only when the caller asks for them); otherwise
  // the logits go to memory and a chunked first stage reads them back
  int groups = 0;
  P0.begin(DFLASH_PROBE_LM_HEAD);
  {
    EpiLogitsTop16<T> et{{seg1<T>(w->lm_head, V, wstride(c, d)), logits, V, STORE}, W.tk_v, W.tk_i};
    groups = run_lm_head_top16<T>(W.ut, d, M, d, V / 16, et, kTopkFinalLists, s, fp8w(c));
    if (groups < 0) return DFLASH_E_HIP;
  }
  // several drafted blocks through the unsplit pipelined LM head: it also leaves each row's
  // maximum per 128-column group, and the top-16 stage reads only the groups that can hold an
  // entry
  const bool by_tiles = groups == 0 && std::is_same<T, bf16_t>::value && (V + 127) / 128 <= 64 * kTopkTilesNG &&
                        pipe_unsplit(M, d, V / 16);
  if (groups == 0) {
    EpiLogits<T> el{{seg1<T>(w->lm_head, V, wstride(c, d)), lg, V, STORE}, by_tiles ? W.tmax : nullptr};
    GEMM_CHECK((run_gemm<T, T>(W.ut, d, nullptr, M, d, V / 16, el, s, W.scratch, W.scratch_bytes, 0, fp8w(c))));
  }
  P0.end(DFLASH_PROBE_LM_HEAD);
  P0.begin(DFLASH_PROBE_TOPK);
  if (by_tiles) {
    topk_tiles_kernel<kTopkTilesNG><<<M, 64, 0, s>>>(lg, V, W.tmax, cand_ids, cand_logits);
    LAUNCH_CHECK();
  } else {
    if (groups == 0) {
      groups = (V + kTopkChunk - 1) / kTopkChunk;
      topk_partial_kernel<<<dim3(groups, M), 64, 0, s>>>(lg, V, V, W.tk_v, W.tk_i);
      LAUNCH_CHECK();
    }
    topk_final_kernel<<<M, 64, 0, s>>>(W.tk_v, W.tk_i, groups, cand_ids, cand_logits);
    LAUNCH_CHECK();
  }
  P0.end(DFLASH_PROBE_TOPK);
  return DFLASH_OK;
}

// ------------------------------------------------------------------ path

template <typename T>
int path_impl(const dflash_config* c, const dflash_weights* w, const int32_t* cand_ids, const float* cand_logits,
              const float* final_hidden, const int32_t* block_ids, int n_fixed, int mode, int B, int32_t* path_idx,
              int32_t* path_ids, float* pair_scores, void* ws, hipStream_t s, float k2 = 0.f,
              const float* uniforms = nullptr, float* path_q = nullptr) {
  Carver cv(ws);
  PathWs W = carve_path<T>(cv, c, B);
  const int d = c->d_model, PD = c->ps_dim, P = c->block_size - n_fixed, Tn = 16 * P + n_fixed;
  const float* table = static_cast<const float*>(w->ps_table);
  if (!table) {   // project the candidates' and the anchor's embeddings now
    path_tokens_kernel<<<B, 256, 0, s>>>(cand_ids, block_ids, n_fixed, P, W.tokens);
    LAUNCH_CHECK();
    SegW<T> sw{};
    sw.p[0] = static_cast<const T*>(w->ps_left);
    sw.p[1] = static_cast<const T*>(w->ps_right);
    sw.off[0] = 0;
    sw.off[1] = PD;
    sw.off[2] = 2 * PD;
    sw.n_seg = 2;
    sw.K = d;
    EpiStore<T> e{sw, W.z, 2 * PD, STORE};
    GEMM_CHECK((run_gemm<T, T>(static_cast<const T*>(w->embed), d, W.tokens, B * Tn, d, 2 * PD / 16, e, s,
                               W.scratch, W.scratch_bytes, c->vocab)));
  }
  if (c->use_gate) {
    EpiStore<T> e{seg1<T>(w->ps_gate, PD, d), W.gamma, PD, SIGMOID};
    bool rounded = false;
    if constexpr (std::is_same<T, bf16_t>::value) rounded = (reinterpret_cast<uintptr_t>(final_hidden) & 15) == 0;
    if (rounded) {
      // the gate reads bf16(x^): rounded once here so the pipelined bf16 kernel applies
      // (256 x 256 x 4096: 31 us on the fp32-input tiled kernel)
      T* xb = static_cast<T*>(W.xb);
      const size_t n4 = static_cast<size_t>(16) * B * d / 4;
      round_to_kernel<T><<<static_cast<unsigned>(std::min<size_t>((n4 + 255) / 256, 2048)), 256, 0, s>>>(
          final_hidden, n4, xb);
      LAUNCH_CHECK();
      GEMM_CHECK((run_gemm<T, T>(xb, d, nullptr, 16 * B, d, PD / 16, e, s, W.scratch, W.scratch_bytes)));
    } else {   // fp32 storage, or rows not 16-byte aligned: A widened/rounded as it is loaded
      GEMM_CHECK((run_gemm<T, float>(final_hidden, d, nullptr, 16 * B, d, PD / 16, e, s, W.scratch,
                                     W.scratch_bytes)));
    }
  }
  const size_t smem = 2 * 16 * (c->ps_rank + 1) * sizeof(float);
  path_scores_kernel<T><<<dim3(P, B), 512, smem, s>>>(W.z, c->use_gate ? W.gamma : nullptr,
                                                      static_cast<const T*>(w->ps_u), static_cast<const T*>(w->ps_v),
                                                      PD, c->ps_rank, n_fixed, P, W.S, pair_scores, table,
                                                      cand_ids, block_ids, c->vocab);
  LAUNCH_CHECK();
  if (uniforms)
    path_sample_kernel<<<B, 64, 0, s>>>(W.S, cand_ids, cand_logits, n_fixed, P, k2, uniforms, path_idx, path_ids,
                                        path_q);
  else
    path_walk_kernel<<<B, 64, 0, s>>>(W.S, cand_ids, cand_logits, n_fixed, P, mode, path_idx, path_ids);
  LAUNCH_CHECK();
  return DFLASH_OK;
}

// ------------------------------------------------------------------ bonus calibration

template <typename T>
int calibrate_impl(const dflash_config* c, const dflash_weights* w, const float* xhat, const int32_t* bonus, int B,
                   float* logits, int32_t* cand_ids, float* cand_logits, void* ws, hipStream_t s) {
  Carver cv(ws);
  CalWs<T> W = carve_cal<T>(cv, c, B);
  const int M = 16 * B, d = c->d_model, C = c->cal_dim, V = c->vocab;
  cal_input_kernel<T><<<M, 256, 0, s>>>(static_cast<const T*>(w->embed), bonus, xhat, d, W.a);
  LAUNCH_CHECK();
  {
    EpiStore<T> e{seg1<T>(w->cal_w1, C, 2 * d), W.h, C, SILU};
    GEMM_CHECK((run_gemm<T, T>(W.a, 2 * d, nullptr, M, 2 * d, C / 16, e, s, W.scratch, W.scratch_bytes)));
  }
  {
    EpiStore<T> e{seg1<T>(w->cal_w2, V, C), logits, V, ADD};
    GEMM_CHECK((run_gemm<T, float>(W.h, C, nullptr, M, C, V / 16, e, s, W.scratch, W.scratch_bytes)));
  }
  const int nch = (V + kTopkChunk - 1) / kTopkChunk;
  topk_partial_kernel<<<dim3(nch, M), 64, 0, s>>>(logits, V, V, W.tk_v, W.tk_i);
  LAUNCH_CHECK();
  topk_final_kernel<<<M, 64, 0, s>>>(W.tk_v, W.tk_i, nch, cand_ids, cand_logits);
  LAUNCH_CHECK();
  return DFLASH_OK;
}

}  // namespace

// ------------------------------------------------------------------ fixed scratch of dflash_verify_noalloc

// Device scratch of the entry point that allocates nothing: one copy per GPU, held by the
// loaded module until the process ends.  In host code `scratch` names a host-side shadow,
// not device memory: the kernels only ever see the address hipGetSymbolAddress returns
// for the current device (noalloc_scratch).
static __device__ __align__(256) unsigned char scratch[DFLASH_VERIFY_NOALLOC_SCRATCH];

namespace {

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, looked up on the first call per
// device with that device current and kept; nullptr when the lookup fails.
void* noalloc_scratch() {
  static std::atomic<void*> addr[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    addr[dev].store(p, std::memory_order_release);
  }
  return p;
}

// Greedy verification over a workspace already carved (shared by both verify entry points).
int verify_launch(const int32_t* draft, const void* tgt_logits, int32_t tgt_dtype, int32_t batch, int32_t n_draft,
                  int32_t vocab, int32_t* accept_len, int32_t* bonus, void* workspace, hipStream_t stream) {
  Carver cv(workspace);
  VerifyWs W = carve_verify(cv, batch, n_draft, vocab);
  const int nch = (vocab + kArgmaxChunk - 1) / kArgmaxChunk;
  dim3 grid(nch, batch * (n_draft + 1));
  if (tgt_dtype == DFLASH_BF16)
    argmax_partial_kernel<bf16_t><<<grid, 256, 0, stream>>>(static_cast<const bf16_t*>(tgt_logits), vocab,
                                                            kArgmaxChunk, W.pv, W.pi);
  else
    argmax_partial_kernel<float><<<grid, 256, 0, stream>>>(static_cast<const float*>(tgt_logits), vocab,
                                                           kArgmaxChunk, W.pv, W.pi);
  LAUNCH_CHECK();
  accept_kernel<<<batch, 64, 0, stream>>>(W.pv, W.pi, nch, draft, n_draft, accept_len, bonus);
  LAUNCH_CHECK();
  return DFLASH_OK;
}

int verify_args(const int32_t* draft, const void* tgt_logits, int32_t tgt_dtype, int32_t batch, int32_t n_draft,
                int32_t vocab, int32_t* accept_len, int32_t* bonus) {
  if (batch <= 0 || n_draft < 0 || vocab <= 0) return DFLASH_E_INVAL;
  if (n_draft > 64) return DFLASH_E_UNSUPPORTED;
  if (tgt_dtype != DFLASH_BF16 && tgt_dtype != DFLASH_F32) return DFLASH_E_INVAL;
  if ((n_draft > 0 && !draft) || !tgt_logits || !accept_len || !bonus) return DFLASH_E_INVAL;
  return DFLASH_OK;
}

}  // namespace

// =====================================================================================
// exported C ABI
// =====================================================================================

extern "C" {

int dflash_check_config(const dflash_config* cfg) { return check_config(cfg); }

const char* dflash_status_string(int status) {
  switch (status) {
    case DFLASH_OK: return "ok";
    case DFLASH_E_INVAL: return "invalid argument";
    case DFLASH_E_UNSUPPORTED: return "unsupported shape";
    case DFLASH_E_WORKSPACE: return "workspace too small";
    case DFLASH_E_CAPACITY: return "KV cache capacity exceeded";
    case DFLASH_E_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

size_t dflash_kv_bytes(const dflash_config* cfg, int32_t batch, int32_t cap) {
  if (check_config(cfg) != DFLASH_OK || batch <= 0 || cap <= 0 || cap % 32 || !kv_slice_ok(cfg, cap)) return 0;
  return static_cast<size_t>(2) * cfg->n_layers * batch * cfg->n_kv_heads * static_cast<size_t>(cap) *
         cfg->head_dim * esize(cfg);
}

size_t dflash_inject_workspace_bytes(const dflash_config* cfg, int32_t n_rows) {
  if (check_config(cfg) != DFLASH_OK || n_rows <= 0) return 0;
  Carver cv(nullptr);
  if (cfg->dtype == DFLASH_BF16) carve_inject<bf16_t>(cv, cfg, n_rows);
  else carve_inject<float>(cv, cfg, n_rows);
  return cv.off;
}

size_t dflash_draft_workspace_bytes(const dflash_config* cfg, int32_t batch, int32_t cap) {
  if (check_config(cfg) != DFLASH_OK || batch <= 0 || cap <= 0) return 0;
  Carver cv(nullptr);
  if (cfg->dtype == DFLASH_BF16) carve_draft<bf16_t>(cv, cfg, batch, cap);
  else carve_draft<float>(cv, cfg, batch, cap);
  return cv.off;
}

size_t dflash_path_workspace_bytes(const dflash_config* cfg, int32_t batch) {
  if (check_config(cfg) != DFLASH_OK || batch <= 0) return 0;
  Carver cv(nullptr);
  if (cfg->dtype == DFLASH_BF16) carve_path<bf16_t>(cv, cfg, batch);
  else carve_path<float>(cv, cfg, batch);
  return cv.off;
}

size_t dflash_verify_workspace_bytes(int32_t batch, int32_t n_draft, int32_t vocab) {
  if (batch <= 0 || n_draft < 0 || n_draft > 64 || vocab <= 0) return 0;
  Carver cv(nullptr);
  carve_verify(cv, batch, n_draft, vocab);
  return cv.off;
}

int dflash_inject_context(const dflash_config* cfg, const dflash_weights* w, const dflash_kv* kv, const void* hidden,
                          int32_t n_rows, const int32_t* row_off, const int32_t* pos0, const int32_t* n_new,
                          int32_t batch, void* workspace, size_t workspace_bytes, const dflash_probes* probes,
                          hipStream_t stream) {
  int rc;
  if ((rc = check_config(cfg))) return rc;
  if ((rc = check_weights(cfg, w, false, true, false))) return rc;
  if (batch <= 0 || n_rows <= 0) return DFLASH_E_INVAL;
  if ((rc = check_kv(cfg, kv, batch))) return rc;
  if (!hidden || !row_off || !pos0 || !n_new || !workspace) return DFLASH_E_INVAL;
  if (workspace_bytes < dflash_inject_workspace_bytes(cfg, n_rows)) return DFLASH_E_WORKSPACE;
  // FP8 storage streams through kernels that address A with 32-bit byte offsets
  if (fp8w(cfg) && static_cast<int64_t>(n_rows) * std::max<int64_t>(cfg->n_feat_layers * int64_t{cfg->d_target},
                                                                      cfg->d_model) * 2 >= (int64_t{1} << 31))
    return DFLASH_E_UNSUPPORTED;
  const Probe pr{probes, stream};
  if (cfg->dtype == DFLASH_BF16)
    return inject_impl<bf16_t>(cfg, w, kv, hidden, n_rows, row_off, pos0, n_new, batch, workspace, pr, stream);
  return inject_impl<float>(cfg, w, kv, hidden, n_rows, row_off, pos0, n_new, batch, workspace, pr, stream);
}

int dflash_draft_block(const dflash_config* cfg, const dflash_weights* w, const dflash_kv* kv, const int32_t* ctx_len,
                       const int32_t* block_ids, int32_t batch, int32_t* cand_ids, float* cand_logits,
                       float* final_hidden, float* logits, void* workspace, size_t workspace_bytes,
                       const dflash_probes* probes, hipStream_t stream) {
  int rc;
  if ((rc = check_config(cfg))) return rc;
  if ((rc = check_weights(cfg, w, true, false, false))) return rc;
  if (batch <= 0) return DFLASH_E_INVAL;
  if ((rc = check_kv(cfg, kv, batch))) return rc;
  if (!ctx_len || !block_ids || !cand_ids || !cand_logits || !final_hidden || !workspace) return DFLASH_E_INVAL;
  if (workspace_bytes < dflash_draft_workspace_bytes(cfg, batch, kv->cap)) return DFLASH_E_WORKSPACE;
  if (fp8w(cfg) && int64_t{16} * batch *
                           std::max<int64_t>({cfg->d_model, int64_t{cfg->n_heads} * cfg->head_dim, cfg->d_ffn}) * 2 >=
                       (int64_t{1} << 31))
    return DFLASH_E_UNSUPPORTED;
  if (cfg->dtype == DFLASH_BF16)
    return draft_impl<bf16_t>(cfg, w, kv, ctx_len, block_ids, batch, cand_ids, cand_logits, final_hidden, logits,
                              workspace, probes, stream);
  return draft_impl<float>(cfg, w, kv, ctx_len, block_ids, batch, cand_ids, cand_logits, final_hidden, logits,
                           workspace, probes, stream);
}

int dflash_select_path(const dflash_config* cfg, const dflash_weights* w, const int32_t* cand_ids,
                       const float* cand_logits, const float* final_hidden, const int32_t* block_ids, int32_t n_fixed,
                       int32_t mode, int32_t batch, int32_t* path_idx, int32_t* path_ids, float* pair_scores,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc;
  if ((rc = check_config(cfg))) return rc;
  if ((rc = check_weights(cfg, w, false, false, true))) return rc;
  if (batch <= 0 || (n_fixed != 0 && n_fixed != 1) || cfg->block_size - n_fixed < 1) return DFLASH_E_INVAL;
  if (mode != DFLASH_PATH_GREEDY && mode != DFLASH_PATH_EXACT) return DFLASH_E_INVAL;
  if (!cand_ids || !cand_logits || !block_ids || !path_idx || !path_ids || !workspace) return DFLASH_E_INVAL;
  if (cfg->use_gate && !final_hidden) return DFLASH_E_INVAL;
  if (workspace_bytes < dflash_path_workspace_bytes(cfg, batch)) return DFLASH_E_WORKSPACE;
  if (cfg->dtype == DFLASH_BF16)
    return path_impl<bf16_t>(cfg, w, cand_ids, cand_logits, final_hidden, block_ids, n_fixed, mode, batch, path_idx,
                             path_ids, pair_scores, workspace, stream);
  return path_impl<float>(cfg, w, cand_ids, cand_logits, final_hidden, block_ids, n_fixed, mode, batch, path_idx,
                          path_ids, pair_scores, workspace, stream);
}

int dflash_verify(const int32_t* draft, const void* tgt_logits, int32_t tgt_dtype, int32_t batch, int32_t n_draft,
                  int32_t vocab, int32_t* accept_len, int32_t* bonus, void* workspace, size_t workspace_bytes,
                  hipStream_t stream) {
  int rc;
  if ((rc = verify_args(draft, tgt_logits, tgt_dtype, batch, n_draft, vocab, accept_len, bonus))) return rc;
  if (!workspace) return DFLASH_E_INVAL;
  if (workspace_bytes < dflash_verify_workspace_bytes(batch, n_draft, vocab)) return DFLASH_E_WORKSPACE;
  return verify_launch(draft, tgt_logits, tgt_dtype, batch, n_draft, vocab, accept_len, bonus, workspace, stream);
}

int dflash_verify_noalloc(const int32_t* draft, const void* tgt_logits, int32_t tgt_dtype, int32_t batch,
                          int32_t n_draft, int32_t vocab, int32_t* accept_len, int32_t* bonus, hipStream_t stream) {
  int rc;
  if ((rc = verify_args(draft, tgt_logits, tgt_dtype, batch, n_draft, vocab, accept_len, bonus))) return rc;
  if (dflash_verify_workspace_bytes(batch, n_draft, vocab) > DFLASH_VERIFY_NOALLOC_SCRATCH) return DFLASH_E_WORKSPACE;
  void* ws = noalloc_scratch();
  if (!ws) return DFLASH_E_HIP;
  return verify_launch(draft, tgt_logits, tgt_dtype, batch, n_draft, vocab, accept_len, bonus, ws, stream);
}

int dflash_sample_path(const dflash_config* cfg, const dflash_weights* w, const int32_t* cand_ids,
                       const float* cand_logits, const float* final_hidden, const int32_t* block_ids, int32_t n_fixed,
                       int32_t batch, float temperature, const float* uniforms, int32_t* path_idx, int32_t* path_ids,
                       float* path_q, float* pair_scores, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  int rc;
  if ((rc = check_config(cfg))) return rc;
  if ((rc = check_weights(cfg, w, false, false, true))) return rc;
  if (batch <= 0 || (n_fixed != 0 && n_fixed != 1) || cfg->block_size - n_fixed < 1) return DFLASH_E_INVAL;
  const float k2 = temp_scale(temperature);
  if (k2 == 0.f) return DFLASH_E_INVAL;
  if (!cand_ids || !cand_logits || !block_ids || !uniforms || !path_idx || !path_ids || !path_q || !workspace)
    return DFLASH_E_INVAL;
  if (cfg->use_gate && !final_hidden) return DFLASH_E_INVAL;
  if (workspace_bytes < dflash_path_workspace_bytes(cfg, batch)) return DFLASH_E_WORKSPACE;
  if (cfg->dtype == DFLASH_BF16)
    return path_impl<bf16_t>(cfg, w, cand_ids, cand_logits, final_hidden, block_ids, n_fixed, DFLASH_PATH_GREEDY,
                             batch, path_idx, path_ids, pair_scores, workspace, stream, k2, uniforms, path_q);
  return path_impl<float>(cfg, w, cand_ids, cand_logits, final_hidden, block_ids, n_fixed, DFLASH_PATH_GREEDY, batch,
                          path_idx, path_ids, pair_scores, workspace, stream, k2, uniforms, path_q);
}

size_t dflash_verify_sampled_workspace_bytes(int32_t batch, int32_t n_draft, int32_t vocab) {
  if (batch <= 0 || n_draft < 0 || n_draft > 64 || vocab <= 0 || vocab > kSoftmaxChunk * 1024) return 0;
  Carver cv(nullptr);
  carve_verify_sampled(cv, batch, n_draft, vocab);
  return cv.off;
}

int dflash_verify_sampled(const int32_t* draft, const int32_t* q_ids, int64_t q_ids_stride, const float* q_probs,
                          const void* tgt_logits, int32_t tgt_dtype, int32_t batch, int32_t n_draft, int32_t vocab,
                          float temperature, const float* u_accept, const float* u_bonus, int32_t* accept_len,
                          int32_t* bonus, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (batch <= 0 || n_draft < 0 || vocab <= 0) return DFLASH_E_INVAL;
  if (n_draft > 64 || vocab > kSoftmaxChunk * 1024) return DFLASH_E_UNSUPPORTED;
  if (tgt_dtype != DFLASH_BF16 && tgt_dtype != DFLASH_F32) return DFLASH_E_INVAL;
  const float k2 = temp_scale(temperature);
  if (k2 == 0.f) return DFLASH_E_INVAL;
  if (n_draft > 0 && (!draft || !q_ids || !q_probs || !u_accept || q_ids_stride < 16LL * n_draft))
    return DFLASH_E_INVAL;
  if (!tgt_logits || !u_bonus || !accept_len || !bonus || !workspace) return DFLASH_E_INVAL;
  if (workspace_bytes < dflash_verify_sampled_workspace_bytes(batch, n_draft, vocab)) return DFLASH_E_WORKSPACE;
  Carver cv(workspace);
  VerifySampledWs W = carve_verify_sampled(cv, batch, n_draft, vocab);
  const int nch = (vocab + kSoftmaxChunk - 1) / kSoftmaxChunk;
  const dim3 grid(nch, batch * (n_draft + 1));
  const long long qs = static_cast<long long>(q_ids_stride);
  if (tgt_dtype == DFLASH_BF16) {
    const bf16_t* T = static_cast<const bf16_t*>(tgt_logits);
    softmax_partial_kernel<bf16_t><<<grid, 256, 0, stream>>>(T, vocab, k2, W.pm, W.ps);
    LAUNCH_CHECK();
    reject_kernel<bf16_t><<<batch, 64, 0, stream>>>(W.pm, W.ps, nch, T, vocab, k2, draft, n_draft, q_ids, qs, q_probs,
                                                     u_accept, u_bonus, accept_len, W.sel);
    LAUNCH_CHECK();
    bonus_kernel<bf16_t><<<batch, 256, 0, stream>>>(T, vocab, k2, n_draft, q_ids, qs, q_probs, W.sel, bonus);
  } else {
    const float* T = static_cast<const float*>(tgt_logits);
    softmax_partial_kernel<float><<<grid, 256, 0, stream>>>(T, vocab, k2, W.pm, W.ps);
    LAUNCH_CHECK();
    reject_kernel<float><<<batch, 64, 0, stream>>>(W.pm, W.ps, nch, T, vocab, k2, draft, n_draft, q_ids, qs, q_probs,
                                                    u_accept, u_bonus, accept_len, W.sel);
    LAUNCH_CHECK();
    bonus_kernel<float><<<batch, 256, 0, stream>>>(T, vocab, k2, n_draft, q_ids, qs, q_probs, W.sel, bonus);
  }
  LAUNCH_CHECK();
  return DFLASH_OK;
}

size_t dflash_path_table_bytes(const dflash_config* cfg) {
  if (check_config(cfg) != DFLASH_OK) return 0;
  return static_cast<size_t>(cfg->vocab) * 2 * cfg->ps_dim * sizeof(float);
}

int dflash_build_path_table(const dflash_config* cfg, const dflash_weights* w, float* table, hipStream_t stream) {
  int rc;
  if ((rc = check_config(cfg))) return rc;
  if (!w || !w->embed || !w->ps_left || !w->ps_right || !table) return DFLASH_E_INVAL;
  const int d = cfg->d_model, PD = cfg->ps_dim, V = cfg->vocab;
  if (cfg->dtype == DFLASH_BF16) {
    SegW<bf16_t> sw{};
    sw.p[0] = static_cast<const bf16_t*>(w->ps_left);
    sw.p[1] = static_cast<const bf16_t*>(w->ps_right);
    sw.off[0] = 0;
    sw.off[1] = PD;
    sw.off[2] = 2 * PD;
    sw.n_seg = 2;
    sw.K = d;
    EpiStore<bf16_t> e{sw, table, 2 * PD, STORE};
    GEMM_CHECK((run_gemm<bf16_t, bf16_t>(static_cast<const bf16_t*>(w->embed), d, nullptr, V, d, 2 * PD / 16, e,
                                         stream)));
  } else {
    SegW<float> sw{};
    sw.p[0] = static_cast<const float*>(w->ps_left);
    sw.p[1] = static_cast<const float*>(w->ps_right);
    sw.off[0] = 0;
    sw.off[1] = PD;
    sw.off[2] = 2 * PD;
    sw.n_seg = 2;
    sw.K = d;
    EpiStore<float> e{sw, table, 2 * PD, STORE};
    GEMM_CHECK((run_gemm<float, float>(static_cast<const float*>(w->embed), d, nullptr, V, d, 2 * PD / 16, e, stream)));
  }
  return DFLASH_OK;
}

size_t dflash_calibrate_workspace_bytes(const dflash_config* cfg, int32_t batch) {
  if (check_config(cfg) != DFLASH_OK || batch <= 0 || cfg->cal_dim <= 0) return 0;
  Carver cv(nullptr);
  if (cfg->dtype == DFLASH_BF16) carve_cal<bf16_t>(cv, cfg, batch);
  else carve_cal<float>(cv, cfg, batch);
  return cv.off;
}

int dflash_calibrate(const dflash_config* cfg, const dflash_weights* w, const float* final_hidden,
                     const int32_t* bonus, int32_t batch, float* logits, int32_t* cand_ids, float* cand_logits,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc;
  if ((rc = check_config(cfg))) return rc;
  if (!w || cfg->cal_dim <= 0 || !w->cal_w1 || !w->cal_w2 || !w->embed) return DFLASH_E_INVAL;
  if (batch <= 0 || !final_hidden || !bonus || !logits || !cand_ids || !cand_logits || !workspace)
    return DFLASH_E_INVAL;
  if (workspace_bytes < dflash_calibrate_workspace_bytes(cfg, batch)) return DFLASH_E_WORKSPACE;
  if (cfg->dtype == DFLASH_BF16)
    return calibrate_impl<bf16_t>(cfg, w, final_hidden, bonus, batch, logits, cand_ids, cand_logits, workspace,
                                  stream);
  return calibrate_impl<float>(cfg, w, final_hidden, bonus, batch, logits, cand_ids, cand_logits, workspace, stream);
}

int dflash_quantize_fp8(const void* w, int32_t rows, int32_t cols, void* out, hipStream_t stream) {
  if (!w || !out || rows <= 0 || cols <= 0 || cols % 64) return DFLASH_E_INVAL;
  if (reinterpret_cast<uintptr_t>(out) % 16) return DFLASH_E_INVAL;
  quantize_fp8_kernel<<<rows, 256, 0, stream>>>(static_cast<const bf16_t*>(w), cols, static_cast<uint8_t*>(out));
  LAUNCH_CHECK();
  return DFLASH_OK;
}

int dflash_advance(const int32_t* accept_len, const int32_t* bonus, int32_t batch, int32_t mask_id, int32_t cap,
                   int32_t* ctx_len, int32_t* pos0, int32_t* n_new, int32_t* block_ids, hipStream_t stream) {
  if (batch <= 0 || cap <= 0 || !accept_len || !bonus || !ctx_len || !pos0 || !n_new || !block_ids)
    return DFLASH_E_INVAL;
  advance_kernel<<<(batch + 63) / 64, 64, 0, stream>>>(accept_len, bonus, batch, mask_id, cap, ctx_len, pos0, n_new,
                                                       block_ids);
  LAUNCH_CHECK();
  return DFLASH_OK;
}

}  // extern "C"
