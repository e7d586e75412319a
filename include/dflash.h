/*
 * dflash.h -- C ABI of one DFlash-style block-diffusion drafting step on an
 * AMD Instinct MI355X (gfx950).
 *
 * The step follows the method as the public descriptions state it:
 *   - "DFlash – Difusión de Bloques para Decodificación Especulativa en Flash"
 *     (gist.science 2602.06036), section 2.2 "Diseño de Inferencia": target hidden
 *     states from several layers are concatenated, projected to one context
 *     feature, pushed through every drafter layer's K/V projections into the
 *     drafter's KV cache; the drafter predicts a whole block of mask tokens in one
 *     forward pass.  Section 2.3: the drafter shares embedding and LM head with
 *     the target; a block starts with a clean anchor token.
 *   - "DFlash 2: optimización de la decodificación especulativa para inferencia
 *     paralela de LLMs" (kerneldigest.dev), "Arquitectura del Sistema": item 1,
 *     the Path Selector (top-16 candidates per position, low-rank bilinear
 *     scoring of adjacent pairs on 256-d embeddings under a context gate, greedy
 *     walk); item 2, the dynamic short convolution (two taps, depthwise,
 *     content-dependent, one correction per 16 channels, before and after every
 *     attention and FFN sublayer); "Flujo de Inferencia con DFlash 2": the target
 *     verifies the chosen block in one pass, accepted tokens are kept.
 *   - "FlexDraft" (gist.science 2605.20022), "Metodología" item 1: mask tokens
 *     attend bidirectionally inside their block and to the clean prefix.
 *
 * Conventions (all calls):
 *   - Every pointer argument named as device memory must point to memory of the
 *     current HIP device; the caller owns it.  The library keeps no pointer to caller
 *     memory after a call returns, and calls on different streams may run concurrently
 *     if they do not share output or workspace memory.  Its only state of its own is
 *     the fixed per-GPU scratch of dflash_verify_noalloc (and that scratch's device
 *     address, looked up once per device).
 *   - Struct arguments (dflash_config, dflash_weights, dflash_kv) are host memory,
 *     read during the call only.
 *   - All device work is enqueued on `stream`; no call synchronises the host or
 *     copies device -> host.  Outputs are valid once the stream reaches them.
 *   - Arguments are validated before anything is enqueued: on a non-zero return
 *     nothing was launched and outputs are untouched.  DFLASH_E_HIP means a launch
 *     failed part-way; outputs are then undefined.
 *   - Linear weights are [out, in] row-major.  Matrices are in the storage type
 *     `cfg->dtype` (bf16 bit patterns or fp32); GEMMs accumulate in fp32.
 *   - Workspace: caller-provided device memory of at least the size the matching
 *     *_workspace_bytes() query returns, 256-byte aligned.  Its content on entry is
 *     irrelevant.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define DFLASH_OK              0
#define DFLASH_E_INVAL        -1   /* null pointer, non-positive size, bad enum value     */
#define DFLASH_E_UNSUPPORTED  -2   /* a shape the kernels do not handle (see each call)   */
#define DFLASH_E_WORKSPACE    -3   /* workspace smaller than the size query returns       */
#define DFLASH_E_CAPACITY     -4   /* host-known sizes exceed the KV cache capacity       */
#define DFLASH_E_HIP          -5   /* a HIP launch failed                                 */

/* storage types */
#define DFLASH_F32   0
#define DFLASH_BF16  1

/* weight storage of the streamed projections (dflash_config.weight_format) */
#define DFLASH_WEIGHTS_DTYPE 0     /* in the storage type dtype                              */
#define DFLASH_WEIGHTS_FP8   1     /* E4M3 codes with a float32 scale per row (bf16 only)    */

/* bytes of one row of a [rows, cols] matrix in FP8 storage */
#define DFLASH_FP8_ROW_BYTES(cols) ((size_t)(cols) + 16)

/* path choice */
#define DFLASH_PATH_GREEDY 0       /* greedy walk over the pair scores (the method's rule) */
#define DFLASH_PATH_EXACT  1       /* maximum total score (dynamic programming)             */

#define DFLASH_MAX_LAYERS 16
#define DFLASH_BLOCK 16            /* rows of a drafted block                               */
#define DFLASH_TOPK  16            /* candidates kept per position                          */
#define DFLASH_CONV_SITES 4        /* conv sites per layer: pre-attn, post-attn, pre-FFN, post-FFN */

typedef struct dflash_config {
  int32_t dtype;          /* DFLASH_BF16 or DFLASH_F32                                        */
  int32_t d_model;        /* drafter width d; multiple of 64                                  */
  int32_t n_heads;        /* query heads H                                                    */
  int32_t n_kv_heads;     /* key/value heads Hkv; H / Hkv in {1, 2, 4}                        */
  int32_t head_dim;       /* 64 or 128                                                        */
  int32_t d_ffn;          /* SwiGLU width; multiple of 64                                     */
  int32_t n_layers;       /* 1 .. DFLASH_MAX_LAYERS                                           */
  int32_t n_feat_layers;  /* sampled target layers n_s                                        */
  int32_t d_target;       /* target width d_t; n_s * d_t multiple of 64                       */
  int32_t vocab;          /* V; multiple of 16, 16 .. 524288                                  */
  int32_t ps_dim;         /* Path Selector embedding width; 256                               */
  int32_t ps_rank;        /* rank r of the bilinear form; 1 .. 256                            */
  int32_t use_conv;       /* 0/1: dynamic short conv around every sublayer                    */
  int32_t use_gate;       /* 0/1: context gate in the Path Selector                           */
  float   rms_eps;        /* RMSNorm epsilon (1e-6)                                           */
  float   rope_theta;     /* rotary base (1e6)                                                */
  int32_t weight_format;  /* DFLASH_WEIGHTS_DTYPE or DFLASH_WEIGHTS_FP8 (see dflash_weights)   */
  int32_t block_size;     /* rows of the drafted block, 1 .. DFLASH_BLOCK (dynamic block size)  */
  int32_t cal_dim;        /* hidden width c of the bonus-calibration MLP; 0: none; else a
                             multiple of 64                                                   */
} dflash_config;

typedef struct dflash_layer_weights {
  const void* w_q;        /* [H*hd, d]                                                        */
  const void* w_k;        /* [Hkv*hd, d]  (used by both inject and draft)                      */
  const void* w_v;        /* [Hkv*hd, d]                                                      */
  const void* w_o;        /* [d, H*hd]                                                        */
  const void* w_gate;     /* [d_ffn, d]                                                       */
  const void* w_up;       /* [d_ffn, d]                                                       */
  const void* w_down;     /* [d, d_ffn]                                                       */
  const void* g_attn;     /* [d] RMSNorm gain before attention                                */
  const void* g_ffn;      /* [d] RMSNorm gain before the FFN                                  */
  const void* conv_gen[DFLASH_CONV_SITES];  /* [2*d/16, d] correction generator (use_conv)    */
  const void* conv_w0[DFLASH_CONV_SITES];   /* [d] static tap on the current row (use_conv)   */
  const void* conv_w1[DFLASH_CONV_SITES];   /* [d] static tap on the previous row (use_conv)  */
} dflash_layer_weights;

/* Weights.  Matrices are row-major [rows, cols] in the storage type, except under
 * weight_format == DFLASH_WEIGHTS_FP8 ("DFlash 2 ...", layer/technology table: draft
 * quantization enabled; bf16 drafters only), where the streamed projections w_fc, w_q,
 * w_k, w_v, w_o, w_gate, w_up, w_down and lm_head are in FP8 storage: row n occupies
 * DFLASH_FP8_ROW_BYTES(cols) = cols + 16 bytes at byte offset n * (cols + 16), holding
 * cols E4M3 codes (the OCP 8-bit format with 4 exponent bits, bias 7, no infinities),
 * then the row's float32 scale, then 12 zero bytes; the row stands for code value times
 * scale.  dflash_quantize_fp8 writes that layout.  The embedding, conv generators and
 * taps, Path Selector factors and norm gains stay in the storage type. */
typedef struct dflash_weights {
  const void* embed;      /* [V, d] token embedding shared with the target                    */
  const void* lm_head;    /* [V, d] LM head shared with the target                            */
  const void* w_fc;       /* [d, n_s*d_t] context-feature projection                          */
  const void* g_fc;       /* [d] RMSNorm gain of the context feature                          */
  const void* g_final;    /* [d] final RMSNorm gain                                           */
  const void* ps_left;    /* [ps_dim, d] left-role projection of token embeddings             */
  const void* ps_right;   /* [ps_dim, d] right-role projection                                 */
  const void* ps_gate;    /* [ps_dim, d] context gate (use_gate)                              */
  const void* ps_u;       /* [r, ps_dim] left factor of the bilinear form                      */
  const void* ps_v;       /* [r, ps_dim] right factor                                          */
  dflash_layer_weights layers[DFLASH_MAX_LAYERS];
  const void* cal_w1;     /* [cal_dim, 2d] bonus-calibration MLP, input layer (cal_dim > 0)    */
  const void* cal_w2;     /* [V, cal_dim]  its output layer                                    */
  const void* ps_table;   /* optional float [V, 2*ps_dim]: every token's embedding projected by
                             ps_left | ps_right (dflash_build_path_table); when set, the Path
                             Selector reads its candidates' rows there instead of projecting
                             their embeddings at each call                                      */
} dflash_weights;

/* The drafter's KV cache of injected context, one pair of arrays per layer.
 *   k[l]  : [batch][Hkv][cap][hd]   keys after RoPE, position-major
 *   vt[l] : [batch][Hkv][hd][cap]   values, transposed (position contiguous)
 * cap is a multiple of 32, and one (sequence, kv head) slice, cap * hd elements, stays
 * below 2 GiB (else DFLASH_E_UNSUPPORTED).  Row p of sequence b holds context position p.
 * Rows at or beyond a sequence's context length are never read by dflash_draft_block. */
typedef struct dflash_kv {
  void*   k[DFLASH_MAX_LAYERS];
  void*   vt[DFLASH_MAX_LAYERS];
  int32_t batch;
  int32_t cap;
} dflash_kv;

/* Optional timing probes.  When a call receives a non-NULL `probes`, it records
 * probes->begin[i] / probes->end[i] (each when non-NULL) on `stream` immediately
 * before the first and after the last launch of stage i.  Per-layer stages are
 * probed on layer 0.  Used to time single kernels inside a running step. */
#define DFLASH_PROBE_LM_HEAD    0   /* draft: LM-head GEMM                          */
#define DFLASH_PROBE_TOPK       1   /* draft: top-16 over the vocabulary            */
#define DFLASH_PROBE_ATTN       2   /* draft: block attention (+ split combine)     */
#define DFLASH_PROBE_QKV        3   /* draft: Q/K/V GEMM with RoPE                  */
#define DFLASH_PROBE_O          4   /* draft: output projection (+ residual)        */
#define DFLASH_PROBE_GATE_UP    5   /* draft: FFN gate/up GEMM with SwiGLU          */
#define DFLASH_PROBE_DOWN       6   /* draft: FFN down projection (+ residual)      */
#define DFLASH_PROBE_INJECT_FC  7   /* inject: context-feature projection GEMM      */
#define DFLASH_PROBE_INJECT_KV  8   /* inject: K/V projection + RoPE + cache scatter */
#define DFLASH_PROBE_CONV_PRE   9   /* draft (use_conv): the FFN input's norm and short conv    */
#define DFLASH_PROBE_CONV_POST 10   /* draft (use_conv): the short conv on the attention output */
#define DFLASH_N_PROBES        11
typedef struct dflash_probes {
  hipEvent_t begin[DFLASH_N_PROBES];
  hipEvent_t end[DFLASH_N_PROBES];
} dflash_probes;

/* Context-feature fusion + KV injection ("DFlash ...", section 2.2).
 *
 * For every new context row r of sequence b (rows row_off[b] .. row_off[b]+n_new[b]-1
 * of `hidden`, i = r - row_off[b] < n_new[b]):
 *   F_r = RMSNorm(hidden_r * w_fc^T; g_fc)            (rounded to the storage type)
 *   k[l][b][:, pos0[b]+i, :]  = RoPE(F_r * w_k^T, pos0[b]+i)   for every layer l
 *   vt[l][b][:, :, pos0[b]+i] = F_r * w_v^T
 *
 * hidden  : device [n_rows, n_s*d_t] storage type, row-major.
 * row_off : device int32 [batch+1], non-decreasing, row_off[batch] <= n_rows.
 * pos0    : device int32 [batch], first cache position written for each sequence.
 * n_new   : device int32 [batch], rows injected; rows of a sequence past n_new[b] are
 *           computed but not written (lets a caller inject accept_len+1 rows of a
 *           fixed 16-row buffer without a host round trip).
 * Rows whose position would reach kv->cap are skipped (never written).
 * n_rows > 0.  Workspace: dflash_inject_workspace_bytes(cfg, n_rows).  probes: NULL or
 * timing probes (see dflash_probes).
 */
int dflash_inject_context(const dflash_config* cfg, const dflash_weights* w, const dflash_kv* kv,
                          const void* hidden, int32_t n_rows, const int32_t* row_off,
                          const int32_t* pos0, const int32_t* n_new, int32_t batch,
                          void* workspace, size_t workspace_bytes, const dflash_probes* probes,
                          hipStream_t stream);

/* One parallel forward pass of the drafter over a 16-row block per sequence
 * ("DFlash ...", sections 2.2-2.3; "DFlash 2 ...", item 2 for the conv).
 *
 * ctx_len   : device int32 [batch], context rows in the cache (0 .. kv->cap).  Block
 *             row j sits at position ctx_len[b] + j.
 * block_ids : device int32 [batch, 16] token ids of the block (anchor and mask ids).
 * Block attention: each block row attends to cache rows 0 .. ctx_len[b]-1 and to all
 * 16 block rows (bidirectional in the block); nothing else.
 * Outputs (device):
 *   cand_ids     int32 [batch, 16, 16]  top-16 token ids per row, best first
 *   cand_logits  float [batch, 16, 16]  their logits (fp32)
 *   final_hidden float [batch, 16, d]   final RMSNorm output (input of the gate)
 *   logits       float [batch, 16, V]   optional (NULL to skip): all logits
 * Order of the top-16: larger logit first, lower id on equal logits.
 * Workspace: dflash_draft_workspace_bytes(cfg, batch, kv->cap).  probes: NULL or timing
 * probes (see dflash_probes).
 */
int dflash_draft_block(const dflash_config* cfg, const dflash_weights* w, const dflash_kv* kv,
                       const int32_t* ctx_len, const int32_t* block_ids, int32_t batch,
                       int32_t* cand_ids, float* cand_logits, float* final_hidden, float* logits,
                       void* workspace, size_t workspace_bytes, const dflash_probes* probes,
                       hipStream_t stream);

/* Path Selector ("DFlash 2 ...", "Arquitectura del Sistema", item 1).
 *
 * Drafted positions are block rows n_fixed..15 (P = 16 - n_fixed); n_fixed is 0 (all
 * rows are mask tokens) or 1 (row 0 is the anchor block_ids[b][0]).  With
 *   z_l(t) = ps_left * E[t],  z_r(t) = ps_right * E[t]                (256-d)
 *   gamma_i = sigmoid(ps_gate * xhat_i)  (use_gate; else 1), xhat_i = final_hidden row i
 *             rounded to the storage type
 *   phi_i(a, t) = (ps_u * z_l(a)) . (ps_v * (gamma_i (.) z_r(t)))
 * the score of candidate j at drafted position p given left token a is
 *   cand_logits[p][j] + phi_{row p}(a, cand_ids[p][j])
 * (no left term at p = 0 without an anchor).  GREEDY walks left to right taking the
 * best score; EXACT maximises the sum over the block.  Ties: lowest candidate index.
 *
 * Inputs: cand_ids int32 [batch,16,16], cand_logits float [batch,16,16],
 *         final_hidden float [batch,16,d], block_ids int32 [batch,16] (device).
 * Outputs: path_idx int32 [batch, P] candidate index per drafted position,
 *          path_ids int32 [batch, P] the chosen token ids,
 *          pair_scores float [batch, P, 16, 16] optional (NULL to skip): phi of every
 *          adjacent candidate pair, [p][a][j] = phi(cand[p-1][a], cand[p][j]); at p = 0
 *          row 0 holds phi(anchor, cand[0][j]) (zeros without anchor), rows 1.. zero.
 * Workspace: dflash_path_workspace_bytes(cfg, batch).
 */
int dflash_select_path(const dflash_config* cfg, const dflash_weights* w,
                       const int32_t* cand_ids, const float* cand_logits, const float* final_hidden,
                       const int32_t* block_ids, int32_t n_fixed, int32_t mode, int32_t batch,
                       int32_t* path_idx, int32_t* path_ids, float* pair_scores,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Greedy verification ("DFlash 2 ...", "Flujo de Inferencia con DFlash 2").
 *
 * draft       : device int32 [batch, n_draft]
 * tgt_logits  : device [batch, n_draft+1, vocab], DFLASH_BF16 or DFLASH_F32 (tgt_dtype);
 *               row i is the target's next-token logits after the draft prefix through i-1.
 * accept_len  : device int32 [batch]: a = number of leading drafts equal to the target's
 *               greedy token of their row.
 * bonus       : device int32 [batch]: the target's greedy token of row a.
 * Greedy token = largest logit, lowest id among equal logits.  n_draft in 0..64.
 * Workspace: dflash_verify_workspace_bytes(batch, n_draft, vocab).
 */
int dflash_verify(const int32_t* draft, const void* tgt_logits, int32_t tgt_dtype, int32_t batch,
                  int32_t n_draft, int32_t vocab, int32_t* accept_len, int32_t* bonus,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Greedy verification that allocates nothing and takes no workspace, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, results and errors as dflash_verify
 * without the workspace.  Its scratch is a fixed array of DFLASH_VERIFY_NOALLOC_SCRATCH
 * bytes inside the library, one copy per GPU, held until the process ends; a call whose
 * dflash_verify_workspace_bytes(batch, n_draft, vocab) exceeds it returns
 * DFLASH_E_WORKSPACE with nothing enqueued (1 MiB covers batch 431 at 15 drafts over a
 * 151,936-token vocabulary).  DFLASH_E_HIP if the scratch's device address cannot be
 * looked up.  Every call on a GPU shares that GPU's array, whose content is whatever the
 * last call left (each call overwrites all of the part it reads, so nothing needs
 * clearing): calls that can overlap on one GPU -- different streams, or host threads
 * without ordering -- race and give undefined results; keep them on one stream. */
#define DFLASH_VERIFY_NOALLOC_SCRATCH (1u << 20)
int dflash_verify_noalloc(const int32_t* draft, const void* tgt_logits, int32_t tgt_dtype, int32_t batch,
                          int32_t n_draft, int32_t vocab, int32_t* accept_len, int32_t* bonus, hipStream_t stream);

/* The Path Selector's per-token table (a cache of weights, not of activations): row t =
 * [ps_left E[t] ; ps_right E[t]] in float (fp32 accumulation), for every token of the
 * vocabulary.  table: device, dflash_path_table_bytes(cfg) bytes.  Needs embed, ps_left,
 * ps_right.  Rebuild it when those weights change. */
size_t dflash_path_table_bytes(const dflash_config* cfg);
int dflash_build_path_table(const dflash_config* cfg, const dflash_weights* w, float* table, hipStream_t stream);

/* Bonus-guided calibration of a drafted block ("FlexDraft", "Metodología" item 2: a
 * light MLP after the LM head turns the resolved bonus token's embedding and a mask
 * position's hidden state into an additive bias of that position's drafted logits, for a
 * block drafted before verification fixed the bonus token).
 *
 * For every row m of sequence b (rows 0..15; rows at or past block_size carry no meaning):
 *   h_m      = silu(cal_w1 [E[bonus[b]] ; bf16(final_hidden_m)])   rounded to the storage type
 *   logits_m += cal_w2 h_m
 * then cand_ids / cand_logits are the top-16 of the calibrated logits (as dflash_draft_block
 * orders them).  cfg->cal_dim > 0 and w->cal_w1, cal_w2, embed set, else DFLASH_E_INVAL.
 *
 * final_hidden : device float [batch, 16, d] (dflash_draft_block's output)
 * bonus        : device int32 [batch]
 * logits       : device float [batch, 16, V] (dflash_draft_block's logits), updated in place
 * cand_ids, cand_logits : device [batch, 16, 16], written.
 * Workspace: dflash_calibrate_workspace_bytes(cfg, batch).
 */
int dflash_calibrate(const dflash_config* cfg, const dflash_weights* w, const float* final_hidden,
                     const int32_t* bonus, int32_t batch, float* logits, int32_t* cand_ids, float* cand_logits,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Sampled path choice ("DFlash 2 ...", "Arquitectura del Sistema", item 1: the block can
 * be chosen by sampling over the precomputed scores instead of the greedy walk).
 *
 * Same scores as dflash_select_path.  Left to right, position p's candidate is drawn from
 *   q_p[j] = softmax_j( (cand_logits[p][j] + phi_{row p}(c_{p-1}, cand_ids[p][j])) / temperature )
 * (no pair term at p = 0 without an anchor): c_p is the first j whose running sum of
 * q_p in candidate order exceeds uniforms[b][p] times the sum of q_p (the last j with
 * q_p[j] > 0 if rounding leaves none).  fp32 throughout.
 *
 * temperature : > 0 and finite (else DFLASH_E_INVAL).
 * uniforms    : device float [batch, P], the caller's uniform draws in [0, 1).
 * path_q      : device float [batch, P, 16], written: q_p, the distribution each position
 *               was drawn from (the proposal that dflash_verify_sampled divides by).
 * Other arguments, outputs and workspace as for dflash_select_path.
 */
int dflash_sample_path(const dflash_config* cfg, const dflash_weights* w,
                       const int32_t* cand_ids, const float* cand_logits, const float* final_hidden,
                       const int32_t* block_ids, int32_t n_fixed, int32_t batch, float temperature,
                       const float* uniforms, int32_t* path_idx, int32_t* path_ids, float* path_q,
                       float* pair_scores, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Verification by rejection sampling, which keeps the target's distribution exactly
 * ("DFlash 2 ...", "Arquitectura del Sistema", item 1; "FlexDraft", problem statement: the
 * bonus token is drawn at the first rejection).
 *
 * p_i = softmax(tgt_logits[b][i] / temperature) over the vocabulary.  Draft token x_i was
 * drawn from the proposal q_i, given sparsely by 16 ids and probabilities (q_i(x) = 0 for
 * ids not listed; ids within a row must be distinct).  Draft i is accepted when
 * u_accept[b][i] * q_i(x_i) < p_i(x_i), i.e. with probability min(1, p_i(x_i) / q_i(x_i));
 * a draft with q_i(x_i) = 0 is rejected.  accept_len[b] = a, the number of leading
 * accepted drafts.  The bonus token is drawn from max(0, p_a - q_a) normalised (from p_a
 * when a = n_draft, or when rounding leaves that residual no mass), inverting its running
 * sum in ascending token id with u_bonus[b].  fp32 exponentials and sums.
 *
 * draft        : device int32 [batch, n_draft]
 * q_ids        : device int32; row i of sequence b at q_ids[b * q_ids_stride + 16 * i + j],
 *                j = 0..15 (q_ids_stride >= 16 * n_draft; the draft call's candidate array
 *                offset by 16 * n_fixed with stride 256 serves directly).
 * q_probs      : device float [batch, n_draft, 16] (dflash_sample_path's path_q).
 * tgt_logits   : device [batch, n_draft+1, vocab], DFLASH_BF16 or DFLASH_F32 (tgt_dtype).
 * u_accept     : device float [batch, n_draft]; u_bonus: device float [batch]; uniforms in [0, 1).
 * accept_len, bonus : device int32 [batch], written.
 * n_draft in 0..64 and vocab <= 4194304 (else DFLASH_E_UNSUPPORTED); temperature > 0 and
 * finite.  Workspace: dflash_verify_sampled_workspace_bytes(batch, n_draft, vocab).
 */
int dflash_verify_sampled(const int32_t* draft, const int32_t* q_ids, int64_t q_ids_stride,
                          const float* q_probs, const void* tgt_logits, int32_t tgt_dtype, int32_t batch,
                          int32_t n_draft, int32_t vocab, float temperature, const float* u_accept,
                          const float* u_bonus, int32_t* accept_len, int32_t* bonus,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Advance the drafting cycle on the device ("DFlash 2 ...", "Flujo de Inferencia con
 * DFlash 2": the verified prefix plus the bonus token are emitted and drafting resumes
 * from them; "DFlash ...", section 2.2: the target's hidden states of the tokens it has
 * processed become new context rows).
 *
 * For a block drafted with an anchor (n_fixed = 1) at position ctx_len[b] and verified
 * with accept_len[b] = a, the target has processed the anchor and the a accepted drafts
 * (positions ctx_len[b] .. ctx_len[b] + a); their hidden states are the next rows to
 * inject, and the bonus token anchors the next block.  Per sequence b:
 *   pos0[b]      = ctx_len[b]
 *   n_new[b]     = a + 1
 *   ctx_len[b]  += a + 1                          (saturating at cap)
 *   block_ids[b] = [bonus[b], mask_id x 15]
 * so the next dflash_inject_context (pos0, n_new) and dflash_draft_block (ctx_len,
 * block_ids) read everything from device memory, with no host synchronisation.
 *
 * accept_len, bonus : device int32 [batch] (dflash_verify's outputs); a is clamped to 0..15.
 * ctx_len           : device int32 [batch], updated in place (clamped to 0..cap first).
 * pos0, n_new       : device int32 [batch], written.
 * block_ids         : device int32 [batch, 16], written.
 * Returns DFLASH_E_INVAL for NULL pointers, batch <= 0 or cap <= 0.  No workspace.
 */
int dflash_advance(const int32_t* accept_len, const int32_t* bonus, int32_t batch, int32_t mask_id, int32_t cap,
                   int32_t* ctx_len, int32_t* pos0, int32_t* n_new, int32_t* block_ids, hipStream_t stream);

/* FP8 storage of one weight matrix (see dflash_weights).
 *
 * w   : device bf16 [rows, cols], row-major.
 * out : device, rows * DFLASH_FP8_ROW_BYTES(cols) bytes, 16-byte aligned; written.
 * Per row: scale = (largest |w|) / 448, code = the E4M3 value nearest to w / scale (both
 * divisions in float32; ties to the even code; magnitudes above 448 saturate); a row of
 * zeros gets scale 0 and codes 0.  rows > 0 and cols a positive multiple of 64, else
 * DFLASH_E_INVAL.  Enqueued on stream; no workspace.
 */
int dflash_quantize_fp8(const void* w, int32_t rows, int32_t cols, void* out, hipStream_t stream);

/* Workspace sizes in bytes (0 when the arguments are invalid). */
size_t dflash_inject_workspace_bytes(const dflash_config* cfg, int32_t n_rows);
size_t dflash_draft_workspace_bytes(const dflash_config* cfg, int32_t batch, int32_t cap);
size_t dflash_path_workspace_bytes(const dflash_config* cfg, int32_t batch);
size_t dflash_verify_workspace_bytes(int32_t batch, int32_t n_draft, int32_t vocab);
size_t dflash_verify_sampled_workspace_bytes(int32_t batch, int32_t n_draft, int32_t vocab);
size_t dflash_calibrate_workspace_bytes(const dflash_config* cfg, int32_t batch);

/* Bytes of a whole KV cache ("DFlash ...", section 2.2: the context features injected
 * into every drafter layer's keys and values) for `batch` sequences of `cap` rows: all
 * 2 * n_layers arrays of dflash_kv, each of them batch * Hkv * cap * hd elements of the
 * storage type (so one array is this size / (2 * n_layers)).  0 when the configuration
 * is invalid, batch <= 0, cap <= 0, cap is not a multiple of 32 or a slice would reach
 * 2 GiB.  The caller allocates the arrays. */
size_t dflash_kv_bytes(const dflash_config* cfg, int32_t batch, int32_t cap);

/* Check a configuration against what the kernels support: DFLASH_OK, DFLASH_E_INVAL
 * or DFLASH_E_UNSUPPORTED. */
int dflash_check_config(const dflash_config* cfg);

/* Static text for a status code. */
const char* dflash_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H */
