"""Plain, slow, obviously-correct CPU oracle of one DFlash-style drafting step.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py``; never by the product path.

Every function follows a passage of the method's public descriptions.  The
pages are cited by title and section:

* [DFlash2] "DFlash 2: optimización de la decodificación especulativa para
  inferencia paralela de LLMs" (kerneldigest.dev), section "Arquitectura del
  Sistema", item 1 (Path Selector) and item 2 (Dynamic Short Convolution);
  section "Flujo de Inferencia con DFlash 2"; its layer/technology table.
* [DFlash] "DFlash – Difusión de Bloques para Decodificación Especulativa en
  Flash" (gist.science 2602.06036), section 2.2 "Diseño de Inferencia" and
  section 2.3 "Estrategia de Entrenamiento".
* [FlexDraft] "FlexDraft" (gist.science 2605.20022), "Metodología", item 1
  "Ajuste de Atención" (mask semantics of a block of mask tokens) and the
  problem statement on the bonus token.
* [Blackwell] "DFlash: Avance en la inferencia de LLM con decodificación
  especulativa en NVIDIA Blackwell", section "Contexto técnico" (accept the
  correct prefix, resume from the last accepted token).

Arithmetic is float64.  Where the GPU contract stores a value in bf16 the
oracle rounds the float64 value to the bf16 grid at exactly that point
(``Model.rb``): weights, target hiddens, the context feature after its norm,
the KV cache (keys after RoPE), and every GEMM input operand (normed / conv'd
activations, the attention output, the SwiGLU product, the final hidden for
the LM head and the gate).  The residual stream, GEMM outputs, logits and
scores stay unrounded.  For the fp32 workload nothing is rounded.

Readings of points the pages leave open are fixed here (and listed with their
reasons in the design notes): pre-norm RMSNorm (eps 1e-6, gain) blocks with
GQA attention and a SwiGLU FFN; rotate-half RoPE with theta 1e6; the fusion
norm; the residual form of the short conv; the Path Selector's factorisation.
Parts whose numbers nothing on the pages fixes (layer internals, RoPE, fusion
norm, Path Selector factorisation) are "parity unpinned" beyond the
invariants the tests check.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

__all__ = [
    "bf16_round", "decode", "Model", "rmsnorm", "rope", "silu", "sigmoid",
    "inject_rows", "short_conv", "block_attention", "draft_block", "topk",
    "path_pair_scores", "select_path", "verify", "conv_param_count",
    "path_selector_param_count", "drafting_step", "advance", "drafting_cycles",
    "sample_path", "verify_sampled", "e4m3_values", "e4m3_encode", "e4m3_decode", "quantize_fp8_rows",
    "dequantize_fp8_rows", "FP8_MATRICES", "is_fp8_matrix", "calibrate",
]


# ----------------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------------

def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored tensor -> float64.  bf16 is given as uint16 bit patterns: the value is the
    float32 whose upper 16 bits are those bits."""
    if dtype == "bf16":
        u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (8 significant bits), ties to even.

    |x| in [2^(e-1), 2^e) has bf16 spacing 2^(e-8); x / spacing is exact in float64 and
    ``np.rint`` rounds half to even.  Values beyond the bf16 range become +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    if fin.any():
        _, e = np.frexp(x[fin])
        e = np.maximum(e, -125)          # below 2^-126 the spacing stays 2^-133 (subnormals)
        ulp = np.ldexp(1.0, e - 8)
        r = np.rint(x[fin] / ulp) * ulp
        big = np.abs(r) >= 2.0 ** 128
        r[big] = np.copysign(np.inf, r[big])
        out[fin] = r
    return out


def e4m3_values() -> np.ndarray:
    """Value of each of the 256 codes of the OCP 8-bit floating-point format E4M3 (the
    "fn" variant: no infinities), float64: bit 7 sign, bits 6..3 exponent with bias 7,
    bits 2..0 mantissa; exponent 0 encodes subnormals m * 2^-9; exponent 15 with
    mantissa 7 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448."""
    v = np.empty(256)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            v[c] = np.nan
        elif e == 0:
            v[c] = sign * m * 2.0 ** -9
        else:
            v[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return v


_E4M3 = e4m3_values()


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Codes of the E4M3 values nearest to x, ties to the even code (even mantissa),
    magnitudes above 448 saturating to +-448; zero (of either sign) encodes as 0.

    In the binade [2^E, 2^(E+1)) the grid spacing is 2^(E-3) (3 mantissa bits); below
    2^-6 it stays 2^-9 (subnormals).  |x| / spacing is exact in float64 and ``np.rint``
    rounds half to even, so the nearest multiple with an even last bit wins ties."""
    x = np.asarray(x)
    if x.dtype != np.float32:        # every step below is exact for float32 inputs
        x = x.astype(np.float64)
    a = np.minimum(np.abs(x), x.dtype.type(448.0))
    _, e = np.frexp(a)                                   # a = f * 2^e, f in [0.5, 1)
    spacing = np.ldexp(x.dtype.type(1.0), np.maximum(e - 1, -6) - 3)
    v = np.minimum(np.rint(a / spacing) * spacing, x.dtype.type(448.0))
    _, e2 = np.frexp(v)
    normal = v >= 2.0 ** -6
    mant = np.where(normal, np.ldexp(v, 4 - e2) - 8, 0)              # v = (8 + mant) * 2^(e2-4)
    code = np.where(normal, (e2 - 1 + 7) * 8 + mant, v * 512).astype(np.uint8)
    neg = (x < 0) & (code != 0)
    return np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def quantize_fp8_rows(w: np.ndarray):
    """Weight quantization to E4M3 with one scale per output row (row of W).

    "DFlash 2 ..." table: the drafter is served with draft quantization enabled.  Reading:
    8-bit E4M3 weights with a float32 scale per output row, the scale being the row's
    largest magnitude over 448 (the format's largest finite value) and each code the E4M3
    value nearest to w / scale; both divisions in float32 (the values the codes are taken
    from are thereby fixed exactly).  A row of zeros gets scale 0 and codes 0.

    w: [rows, cols] float32 (the stored bf16 weights, decoded).  Returns (codes uint8
    [rows, cols], scales float32 [rows]).
    """
    w = np.asarray(w, dtype=np.float32)
    amax = np.abs(w).max(axis=1).astype(np.float32)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    codes = np.empty(w.shape, dtype=np.uint8)
    for r0 in range(0, w.shape[0], 2048):                 # row blocks bound the temporaries
        x = (w[r0:r0 + 2048] / safe[r0:r0 + 2048, None]).astype(np.float32)
        codes[r0:r0 + 2048] = e4m3_encode(x)
    codes[scale == 0] = 0
    return codes, scale


def dequantize_fp8_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """The weights an E4M3 matrix stands for: code value times its row's scale (float64)."""
    return e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[:, None]


# Weights held in E4M3 under fp8 weight storage: every streamed projection of the drafter
# (fusion, Q/K/V, O, gate/up, down, LM head).  The token embedding (gathered by rows), the
# dynamic-conv generators and taps, the Path Selector's factors and the norm gains stay in
# the storage type.
FP8_MATRICES = ("w_fc", "lm_head", "w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down")


def is_fp8_matrix(name: str) -> bool:
    return name.split(".")[-1] in FP8_MATRICES


# ----------------------------------------------------------------------------------
# model container
# ----------------------------------------------------------------------------------

class Model:
    """Weights of one drafter, decoded to float64 on first use and kept.

    ``dims`` carries the sizes (any object with the attributes of ``synth.Dims``);
    ``weights`` maps names to stored tensors (bf16 bit patterns or float32).
    """

    def __init__(self, dims, weights: Dict[str, np.ndarray], fp8: bool = False):
        if fp8 and dims.dtype != "bf16":
            raise ValueError("fp8 weight storage applies to bf16 drafters")
        self.dims = dims
        self.stored = weights
        self.fp8 = fp8
        self._cache: Dict[str, np.ndarray] = {}

    def w(self, name: str) -> np.ndarray:
        """Weight values as float64; under fp8 storage the projections listed in
        ``FP8_MATRICES`` are the values their E4M3 codes and row scales stand for."""
        if name not in self._cache:
            v = decode(self.stored[name], self.dims.dtype)
            if self.fp8 and is_fp8_matrix(name):
                v = dequantize_fp8_rows(*quantize_fp8_rows(v.astype(np.float32)))
            self._cache[name] = v
        return self._cache[name]

    def rows(self, name: str, idx) -> np.ndarray:
        """Rows ``idx`` of a weight matrix (used for embedding gathers)."""
        if name in self._cache:
            return self._cache[name][idx]
        return decode(self.stored[name][idx], self.dims.dtype)

    def rb(self, x: np.ndarray) -> np.ndarray:
        """Round to the storage type at a contract point (identity for fp32 workloads)."""
        return bf16_round(x) if self.dims.dtype == "bf16" else np.asarray(x, dtype=np.float64)


# ----------------------------------------------------------------------------------
# building blocks
# ----------------------------------------------------------------------------------

def rmsnorm(v: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """Root-mean-square norm over the last axis, then the per-channel gain."""
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v / np.sqrt(ms + eps) * g


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary position encoding, rotate-half pairing.

    ``x`` is ``[n, heads, hd]`` and ``pos`` ``[n]``.  Dimension i < hd/2 is paired with
    i + hd/2 and the pair is rotated by the angle pos * theta^(-2i/hd).
    """
    hd = x.shape[-1]
    half = hd // 2
    inv = theta ** (-2.0 * np.arange(half, dtype=np.float64) / hd)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]          # [n, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


# ----------------------------------------------------------------------------------
# (a1, a2) context feature and KV injection
# ----------------------------------------------------------------------------------

def inject_rows(m: Model, hidden: np.ndarray, pos: np.ndarray):
    """Context-feature fusion and KV injection for one sequence's new context rows.

    [DFlash] section 2.2: hidden states taken from several target layers are
    concatenated per context row and projected to one compact context feature;
    that feature goes through the Key and Value projections of every drafter
    layer and the results are kept in the drafter's KV cache.

    ``hidden`` is ``[n, n_feat_layers * d_target]`` (stored bits/fp32), ``pos`` the
    cache positions of the rows.  Returns ``(F, K, V)``: the feature ``[n, d]`` and,
    per layer, keys after RoPE and values, ``[L, n, Hkv, hd]``, all rounded to the
    cache type.
    """
    D = m.dims
    H = decode(hidden, D.dtype)                                   # already on the storage grid
    F = m.rb(rmsnorm(H @ m.w("w_fc").T, m.w("g_fc"), D.rms_eps))
    n = H.shape[0]
    Ks, Vs = [], []
    for l in range(D.n_layers):
        k = (F @ m.w(f"l{l}.w_k").T).reshape(n, D.n_kv_heads, D.head_dim)
        v = (F @ m.w(f"l{l}.w_v").T).reshape(n, D.n_kv_heads, D.head_dim)
        Ks.append(m.rb(rope(k, pos, D.rope_theta)))
        Vs.append(m.rb(v))
    return F, np.stack(Ks), np.stack(Vs)


# ----------------------------------------------------------------------------------
# (a8) DFlash 2 dynamic short convolution
# ----------------------------------------------------------------------------------

def conv_site_shapes(d: int) -> Dict[str, tuple]:
    """Parameters of one conv site: the correction generator (one correction per group of
    16 channels, for each of the two taps) and the two static per-channel taps."""
    return {"gen": (2 * (d // 16), d), "w0": (d,), "w1": (d,)}


def conv_param_count(d: int, n_layers: int, sites_per_layer: int = 4) -> int:
    return n_layers * sites_per_layer * sum(int(np.prod(s)) for s in conv_site_shapes(d).values())


def short_conv(m: Model, layer: int, site: int, u: np.ndarray) -> np.ndarray:
    """Two-tap depthwise convolution along the block with content-dependent taps.

    [DFlash2] "Arquitectura del Sistema", item 2: one tap on the current position and
    one on the previous position, depthwise; the coefficients adapt to the current
    hidden state, with one correction shared by each group of 16 channels; local to
    the block and stateless.  Readings: the corrections are a linear map of the current
    row added to static per-channel taps, and the conv is residual, so zero taps and a
    zero generator give the identity.  Row 0 of the block has no previous row (zero).

    ``u`` is ``[16, d]`` float64.
    """
    D = m.dims
    d = D.d
    ng = d // 16
    p = f"l{layer}.conv{site}."
    gen, w0, w1 = m.w(p + "gen"), m.w(p + "w0"), m.w(p + "w1")
    assert gen.shape == conv_site_shapes(d)["gen"]
    delta = m.rb(u) @ gen.T                                   # [16, 2*ng]
    a = w0[None, :] + np.repeat(delta[:, :ng], 16, axis=1)     # channel c uses group c // 16
    b = w1[None, :] + np.repeat(delta[:, ng:], 16, axis=1)
    u_prev = np.vstack([np.zeros((1, d)), u[:-1]])
    return u + a * u + b * u_prev


# ----------------------------------------------------------------------------------
# (a5) block attention
# ----------------------------------------------------------------------------------

def block_attention(q: np.ndarray, k_ctx: np.ndarray, v_ctx: np.ndarray,
                    k_blk: np.ndarray, v_blk: np.ndarray) -> np.ndarray:
    """Attention of the block's queries over the injected context and the block itself.

    [DFlash] section 2.2 (the whole block is predicted in one forward pass over the
    persistent context) and [FlexDraft] "Metodología" item 1 (mask tokens attend
    bidirectionally inside their block and to the clean prefix): every block row sees
    every context row and every block row, with no mask among them.

    q: [16, H, hd]; k_ctx, v_ctx: [Hkv, L, hd]; k_blk, v_blk: [16, Hkv, hd].
    Query head h reads key/value head h // (H / Hkv).  Returns [16, H, hd].
    """
    nq, H, hd = q.shape
    Hkv = k_ctx.shape[0]
    group = H // Hkv
    out = np.empty_like(q)
    for h in range(H):
        g = h // group
        keys = np.concatenate([k_ctx[g], k_blk[:, g]], axis=0)
        vals = np.concatenate([v_ctx[g], v_blk[:, g]], axis=0)
        s = q[:, h] @ keys.T / math.sqrt(hd)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h] = p @ vals
    return out


# ----------------------------------------------------------------------------------
# (a3..a9) drafter forward over one block
# ----------------------------------------------------------------------------------

def draft_block(m: Model, k_cache: Sequence[np.ndarray], v_cache: Sequence[np.ndarray],
                ctx_len: int, block_ids: np.ndarray) -> Dict[str, np.ndarray]:
    """One parallel forward pass of the drafter over a block of up to 16 tokens.

    [DFlash] section 2.2: the block (a clean anchor followed by mask tokens, section 2.3)
    is predicted in a single forward pass; every layer attends to the injected context
    in its KV cache.  [DFlash] section 2.3: token embedding and LM head are shared with
    the target.  [DFlash2] item 2: with the conv enabled, a short conv sits before and
    after the attention and the FFN sublayer of every layer.

    k_cache, v_cache: per layer ``[Hkv, >=ctx_len, hd]`` float64 (rows beyond ctx_len are
    never read).  block_ids: [nb] ints, nb = 16 or, under dynamic block-size scheduling,
    fewer ([DFlash] sections 3 and 4: a drafter trained on blocks of 16 drafts smaller
    blocks at inference; the block is then just nb rows).  Positions: context rows
    0..ctx_len-1, block rows ctx_len..ctx_len+nb-1.  Returns the fp64 logits ``[nb, V]``,
    the final normed hidden ``xhat [nb, d]`` and per-layer residual streams.
    """
    D = m.dims
    nb = len(block_ids)
    pos = ctx_len + np.arange(nb)
    x = m.rows("embed", np.asarray(block_ids))                 # [16, d]
    stream = [x.copy()]
    for l in range(D.n_layers):
        p = f"l{l}."
        # attention sublayer
        u = rmsnorm(x, m.w(p + "g_attn"), D.rms_eps)
        if D.use_conv:
            u = short_conv(m, l, 0, u)
        u = m.rb(u)
        q = (u @ m.w(p + "w_q").T).reshape(nb, D.n_heads, D.head_dim)
        k = (u @ m.w(p + "w_k").T).reshape(nb, D.n_kv_heads, D.head_dim)
        v = (u @ m.w(p + "w_v").T).reshape(nb, D.n_kv_heads, D.head_dim)
        q = m.rb(rope(q, pos, D.rope_theta))
        k = m.rb(rope(k, pos, D.rope_theta))
        v = m.rb(v)
        kc = k_cache[l][:, :ctx_len]
        vc = v_cache[l][:, :ctx_len]
        o = m.rb(block_attention(q, kc, vc, k, v).reshape(nb, D.n_heads * D.head_dim))
        a = o @ m.w(p + "w_o").T
        if D.use_conv:
            a = short_conv(m, l, 1, a)
        x = x + a
        # feed-forward sublayer (SwiGLU)
        u = rmsnorm(x, m.w(p + "g_ffn"), D.rms_eps)
        if D.use_conv:
            u = short_conv(m, l, 2, u)
        u = m.rb(u)
        h = m.rb(silu(u @ m.w(p + "w_gate").T) * (u @ m.w(p + "w_up").T))
        f = h @ m.w(p + "w_down").T
        if D.use_conv:
            f = short_conv(m, l, 3, f)
        x = x + f
        stream.append(x.copy())
    xhat = rmsnorm(x, m.w("g_final"), D.rms_eps)
    logits = m.rb(xhat) @ m.w("lm_head").T
    return {"logits": logits, "xhat": xhat, "stream": stream}


def topk(logits: np.ndarray, k: int = 16):
    """The k best entries of each row, ordered by (value descending, id ascending).

    [DFlash2] item 1: the drafter keeps the 16 best candidates per position.  The order
    is decided on float32 values (the precision the device keeps logits in).
    Returns (ids int32 [..., k], values float32 [..., k]).
    """
    lg = np.asarray(logits, dtype=np.float64).astype(np.float32)
    flat = lg.reshape(-1, lg.shape[-1])
    ids = np.empty((flat.shape[0], k), dtype=np.int32)
    for r in range(flat.shape[0]):
        taken = np.zeros(flat.shape[1], dtype=bool)
        for t in range(k):                     # pick the best remaining entry k times
            best = _argmax_lowest(np.where(taken, -np.inf, flat[r]), exclude=taken)
            ids[r, t] = best
            taken[best] = True
    vals = np.take_along_axis(flat, ids.astype(np.int64), axis=1)
    return ids.reshape(lg.shape[:-1] + (k,)), vals.reshape(lg.shape[:-1] + (k,))


# ----------------------------------------------------------------------------------
# (a10) Path Selector
# ----------------------------------------------------------------------------------

def path_selector_param_count(d: int, ps_dim: int, rank: int, gate: bool = True) -> int:
    """Left and right projections of the token embedding to ``ps_dim``, the context gate
    (``ps_dim`` x d) and the two rank-``rank`` factors of the bilinear form."""
    return (3 if gate else 2) * ps_dim * d + 2 * rank * ps_dim


def path_pair_scores(m: Model, cand_ids: np.ndarray, xhat: np.ndarray, block_ids: np.ndarray,
                     n_fixed: int) -> np.ndarray:
    """Compatibility scores of every adjacent candidate pair, for one sequence.

    [DFlash2] item 1: each pair of candidates at adjacent positions is scored by a
    low-rank bilinear form over 256-d token embeddings, under a context gate; all pairs
    are scored at once.  Readings: the 256-d embeddings are two learned projections of
    the shared token embedding (left and right roles); the gate is a sigmoid of a linear
    map of the right position's final hidden state; the bilinear form is rank r:
        phi_i(a, b) = (U z_l(a)) . (V (gamma_i * z_r(b))).

    cand_ids: [>=nb, 16] candidates per block row; xhat: [>=nb, d]; block_ids: [nb] (nb =
    the block size).  Drafted positions are rows n_fixed..nb-1, renumbered p = 0..P-1.  Returns S [P, 16, 16]:
    for p >= 1, S[p, a, j] = phi(cand[p-1][a], cand[p][j]); for p = 0 row a = 0 holds
    phi(anchor, cand[0][j]) when there is an anchor (n_fixed = 1), everything else 0.
    """
    D = m.dims
    nb = len(block_ids)
    P = nb - n_fixed
    K = cand_ids.shape[-1]
    Pl, Pr = m.w("ps_left"), m.w("ps_right")
    U, Vf = m.w("ps_u"), m.w("ps_v")
    rows = np.arange(n_fixed, nb)
    cands = np.asarray(cand_ids)[rows]                                 # [P, K]
    if D.use_gate:
        gamma = sigmoid(m.rb(np.asarray(xhat, dtype=np.float64)[rows]) @ m.w("ps_gate").T)   # [P, 256]
    else:
        gamma = np.ones((P, Pl.shape[0]))

    def lam(tokens):                     # left factor of each token: [n, r]
        return (m.rows("embed", tokens) @ Pl.T) @ U.T

    def rho(p, tokens):                  # right factor at drafted position p: [n, r]
        return (gamma[p][None, :] * (m.rows("embed", tokens) @ Pr.T)) @ Vf.T

    S = np.zeros((P, K, K))
    if n_fixed == 1:
        S[0, 0, :] = lam(np.asarray([block_ids[0]])) @ rho(0, cands[0]).T
    for p in range(1, P):
        S[p] = lam(cands[p - 1]) @ rho(p, cands[p]).T
    return S


def select_path(cand_logits: np.ndarray, S: np.ndarray, has_anchor: bool, mode: str = "greedy"):
    """Choose one candidate per drafted position.

    [DFlash2] item 1: the final sequence is picked by a greedy walk over the precomputed
    scores (the score of a candidate is its drafter logit plus its compatibility with
    the chosen left neighbour).  ``mode="exact"`` maximises the total score over all
    paths (dynamic programming), the yardstick the greedy walk is measured against.
    Ties go to the lowest candidate index.

    cand_logits: [P, K]; S: [P, K, K] as from ``path_pair_scores``.  Returns
    (indices [P] int32, total score float).
    """
    lg = np.asarray(cand_logits, dtype=np.float64)
    P, K = lg.shape
    first = lg[0] + (S[0, 0] if has_anchor else 0.0)
    if mode == "greedy":
        idx = [int(np.argmax(first))]
        total = float(first[idx[0]])
        for p in range(1, P):
            sc = lg[p] + S[p, idx[-1]]
            j = int(np.argmax(sc))           # argmax returns the first maximum
            idx.append(j)
            total += float(sc[j])
        return np.asarray(idx, dtype=np.int32), total
    if mode == "exact":
        best = first.copy()
        back = np.zeros((P, K), dtype=np.int64)
        for p in range(1, P):
            cand = best[:, None] + S[p]                     # [prev a, next j]
            back[p] = np.argmax(cand, axis=0)
            best = lg[p] + cand[back[p], np.arange(K)]
        j = int(np.argmax(best))
        total = float(best[j])
        idx = [j]
        for p in range(P - 1, 0, -1):
            j = int(back[p, j])
            idx.append(j)
        return np.asarray(idx[::-1], dtype=np.int32), total
    raise ValueError(mode)


def sample_path(cand_logits: np.ndarray, S: np.ndarray, has_anchor: bool, temperature: float,
                uniforms: np.ndarray):
    """Draw one candidate per drafted position from the precomputed scores.

    [DFlash2] item 1 names sampling over the precomputed scores as the alternative to the
    greedy walk.  Reading: left to right, the candidate at position p is drawn from the
    softmax, at the given temperature, of the very scores the greedy walk maximises
    (drafter logit plus compatibility with the candidate drawn at p - 1; the anchor, or
    nothing, at p = 0).  Each draw inverts the cumulative distribution in candidate-index
    order with the uniform ``uniforms[p]`` in [0, 1): the first j whose cumulative
    probability exceeds u (the last candidate of non-zero probability if rounding leaves
    u above the total).

    cand_logits: [P, K]; S: [P, K, K] as from ``path_pair_scores``; temperature > 0.
    Returns (indices [P] int32, q [P, K]) where q[p] is the distribution position p was
    drawn from: the proposal distribution that rejection sampling divides by.
    """
    lg = np.asarray(cand_logits, dtype=np.float64)
    P, K = lg.shape
    t = float(temperature)
    if not t > 0:
        raise ValueError("temperature must be positive")
    idx = np.zeros(P, dtype=np.int32)
    q = np.zeros((P, K))
    prev = None
    for p in range(P):
        if p == 0:
            sc = lg[0] + (S[0, 0] if has_anchor else 0.0)
        else:
            sc = lg[p] + S[p, prev]
        w = np.exp((sc - sc.max()) / t)
        q[p] = w / w.sum()
        idx[p] = _inverse_cdf(q[p], float(uniforms[p]))
        prev = idx[p]
    return idx, q


def _inverse_cdf(w: np.ndarray, u: float) -> int:
    """First index whose running sum of the non-negative weights ``w`` exceeds u * sum(w);
    the last index of positive weight if none does (rounding at the top end)."""
    w = np.asarray(w, dtype=np.float64)
    target = u * w.sum()
    run = 0.0
    for i, wi in enumerate(w):
        run += wi
        if target < run:
            return i
    return int(np.flatnonzero(w > 0)[-1])


# ----------------------------------------------------------------------------------
# bonus-guided calibration of the drafted logits
# ----------------------------------------------------------------------------------

def calibrate(m: Model, xhat: np.ndarray, bonus: int, logits: np.ndarray) -> np.ndarray:
    """Logits of a drafted block after bonus-guided calibration.

    [FlexDraft] "Calibración Guiada por Bono": a light MLP after the LM head takes the
    concatenation of the resolved bonus token's embedding and the hidden state of a mask
    position and returns an additive bias for that position's drafted logits (the block
    was drafted before verification had fixed the bonus token).  Reading: one hidden layer
    of width c with SiLU and no biases,
        bias_i = W2 bf16(silu(W1 [bf16(E[bonus]); bf16(xhat_i)])),
    W1 [c, 2d] ("cal_w1"), W2 [V, c] ("cal_w2"); the hidden state is the final normed
    hidden state the LM head reads; the bias is added to the fp32 logits.

    xhat: [nb, d]; logits: [nb, V].  Returns the calibrated logits [nb, V] (float64).
    """
    x = np.asarray(xhat, dtype=np.float64)
    e = m.rows("embed", np.asarray([int(bonus)]))[0]
    a = np.concatenate([np.broadcast_to(m.rb(e), x.shape), m.rb(x)], axis=1)    # [nb, 2d]
    h = m.rb(silu(a @ m.w("cal_w1").T))
    return np.asarray(logits, dtype=np.float64) + h @ m.w("cal_w2").T


# ----------------------------------------------------------------------------------
# (a11) greedy verification
# ----------------------------------------------------------------------------------

def verify(draft: np.ndarray, target_logits: np.ndarray):
    """Greedy acceptance of one drafted block.

    [DFlash2] "Flujo de Inferencia": the target checks the chosen block in one pass;
    accepted tokens are appended and the rest discarded.  [Blackwell] "Contexto
    técnico": the correct prefix is kept and generation resumes from the last accepted
    token.  [FlexDraft] problem statement: the bonus token is the target's own token at
    the first rejection.  Row i of the target logits is the target's next-token
    distribution after the block prefix through draft i-1.

    draft: [P] ints; target_logits: [P+1, V] floats (ties resolve to the lowest id).
    Returns (accepted length a, bonus token) with a = number of leading drafts equal to
    the target's greedy token and bonus = the target's greedy token at row a.
    """
    P = len(draft)
    a = 0
    while a < P:
        best = _argmax_lowest(target_logits[a])
        if int(draft[a]) != best:
            break
        a += 1
    return a, _argmax_lowest(target_logits[a])


def verify_sampled(draft: np.ndarray, q_ids: np.ndarray, q_probs: np.ndarray, target_logits: np.ndarray,
                   temperature: float, u_accept: np.ndarray, u_bonus: float):
    """Verification by rejection sampling, which keeps the target's distribution exactly.

    [DFlash2] item 1: besides the greedy walk, the block can be chosen so that rejection
    sampling restores the target model's exact distribution; [FlexDraft] problem
    statement: the bonus token is drawn at the first rejection.  Reading (speculative
    sampling in its standard form): the target's distribution at row i is
    p_i = softmax(target_logits[i] / temperature); draft token x_i was drawn from the
    proposal q_i, given sparsely by (q_ids[i], q_probs[i]) (q_i(x) = 0 for ids not listed).
    Draft i is accepted with probability min(1, p_i(x_i) / q_i(x_i)), decided as
    u_accept[i] * q_i(x_i) < p_i(x_i) (a draft with q_i(x_i) = 0 is rejected).  At the first
    rejection a the bonus token is drawn from the residual max(0, p_a - q_a), normalised;
    if every draft is accepted (a = P) it is drawn from p_P.  The draw inverts the
    cumulative distribution in ascending token id with u_bonus.  If the residual has no
    positive mass (possible only through rounding) the bonus is drawn from p_a.

    draft: [P]; q_ids, q_probs: [P, K]; target_logits: [P+1, V]; u_accept: [P]; u_bonus
    scalar, uniforms in [0, 1).  Returns (accepted length a, bonus token).
    """
    t = float(temperature)
    if not t > 0:
        raise ValueError("temperature must be positive")
    T = np.asarray(target_logits, dtype=np.float64)
    P = len(draft)

    def probs(row):
        z = (T[row] - T[row].max()) / t
        w = np.exp(z)
        return w / w.sum()

    a = 0
    while a < P:
        x = int(draft[a])
        hit = np.flatnonzero(np.asarray(q_ids[a]) == x)
        q = float(q_probs[a][hit[0]]) if len(hit) else 0.0
        if not (q > 0.0 and float(u_accept[a]) * q < probs(a)[x]):
            break
        a += 1
    p = probs(a)
    r = p.copy()
    if a < P:
        ids = np.asarray(q_ids[a])
        r[ids] = np.maximum(0.0, p[ids] - np.asarray(q_probs[a], dtype=np.float64))
    if not r.sum() > 0.0:
        r = p
    return a, _inverse_cdf(r, float(u_bonus))


def _argmax_lowest(row: np.ndarray, exclude: Optional[np.ndarray] = None) -> int:
    """Index of the largest entry; among equal largest entries the lowest index."""
    row = np.asarray(row)
    ok = np.ones(row.shape, dtype=bool) if exclude is None else ~exclude
    m = row[ok].max()
    return int(np.flatnonzero(ok & (row == m))[0])


# ----------------------------------------------------------------------------------
# one whole step (used by the CPU baseline and the end-to-end tests)
# ----------------------------------------------------------------------------------

def drafting_step(m: Model, k_cache: List[np.ndarray], v_cache: List[np.ndarray], ctx_len: int,
                  new_hidden: np.ndarray, new_pos: np.ndarray, block_ids: np.ndarray,
                  target_logits: np.ndarray, n_fixed: int = 1, mode: str = "greedy"):
    """Inject new context rows, draft a block, choose a path, verify it: one sequence.

    k_cache/v_cache: per layer float64 ``[Hkv, cap, hd]``, updated in place at ``new_pos``.
    Returns a dict with the step's outputs.
    """
    D = m.dims
    if len(new_pos):
        _, K, V = inject_rows(m, new_hidden, np.asarray(new_pos))
        for l in range(D.n_layers):
            k_cache[l][:, new_pos] = np.transpose(K[l], (1, 0, 2))
            v_cache[l][:, new_pos] = np.transpose(V[l], (1, 0, 2))
    out = draft_block(m, k_cache, v_cache, ctx_len, block_ids)
    ids, vals = topk(out["logits"], D.topk)
    S = path_pair_scores(m, ids, out["xhat"], block_ids, n_fixed)
    idx, _ = select_path(vals[n_fixed:], S, n_fixed == 1, mode)
    path_ids = ids[np.arange(n_fixed, len(block_ids)), idx]
    a, bonus = verify(path_ids, target_logits)
    return {"cand_ids": ids, "cand_logits": vals, "xhat": out["xhat"], "logits": out["logits"],
            "pair_scores": S, "path_idx": idx, "path_ids": path_ids, "accept_len": a, "bonus": bonus}


# --------------------------------------------------------------------------------------
# the drafting cycle (draft -> verify -> inject)
# --------------------------------------------------------------------------------------

def advance(accept_len: int, bonus: int, ctx_len: int, mask_id: int, cap: int, block: int = 16):
    """State of the next cycle after a block drafted with an anchor at position ctx_len was
    verified ("DFlash 2 ...", inference flow: the accepted prefix and the bonus token are
    emitted and drafting resumes from them; "DFlash ...", section 2.2: the target's hidden
    states of the tokens it processed become new context rows).  The target processed the
    anchor and the a accepted drafts, positions ctx_len .. ctx_len + a: those a + 1 rows are
    injected next, and the bonus token anchors the next block.  a is clamped to
    0 .. block - 1 and ctx_len to 0 .. cap; the new ctx_len saturates at cap."""
    a = min(max(int(accept_len), 0), block - 1)
    L = min(max(int(ctx_len), 0), cap)
    ids = np.full(block, mask_id, dtype=np.int32)
    ids[0] = bonus
    return {"pos0": L, "n_new": a + 1, "ctx_len": min(L + a + 1, cap), "block_ids": ids}


def drafting_cycles(m: Model, k_cache: List[np.ndarray], v_cache: List[np.ndarray], ctx_len: int, cap: int,
                    pos0: int, n_new: int, block_ids: np.ndarray, hidden_fn, logits_fn, cycles: int,
                    mode: str = "greedy"):
    """``cycles`` drafting cycles of one sequence.  Each cycle injects n_new rows at pos0
    (``hidden_fn(c, n)`` gives the target's hidden states of those rows, stored values as
    for ``inject_rows``; rows at positions >= cap are dropped), drafts the block anchored by block_ids[0], chooses the path,
    verifies it against ``logits_fn(c, path_ids)`` (the target's logits for the block),
    emits the accepted drafts and the bonus token, and advances.  k_cache/v_cache are
    updated in place.  Returns one dict per cycle."""
    D = m.dims
    out = []
    for c in range(cycles):
        pos = pos0 + np.arange(n_new)
        keep = pos < cap
        if keep.any():
            rows = np.asarray(hidden_fn(c, n_new))[keep]
            _, K, V = inject_rows(m, rows, pos[keep])
            for l in range(D.n_layers):
                k_cache[l][:, pos[keep]] = np.transpose(K[l], (1, 0, 2))
                v_cache[l][:, pos[keep]] = np.transpose(V[l], (1, 0, 2))
        d = draft_block(m, k_cache, v_cache, min(ctx_len, cap), block_ids)
        ids, vals = topk(d["logits"], D.topk)
        S = path_pair_scores(m, ids, d["xhat"], block_ids, 1)
        idx, _ = select_path(vals[1:], S, True, mode)
        path_ids = ids[np.arange(1, len(block_ids)), idx]
        T = logits_fn(c, path_ids)
        a, bonus = verify(path_ids, T)
        nxt = advance(a, bonus, ctx_len, D.mask_id, cap, len(block_ids))
        out.append({"cand_ids": ids, "logits": d["logits"], "path_ids": path_ids, "target_logits": T,
                    "accept_len": a, "bonus": bonus, "emitted": list(path_ids[:a]) + [bonus],
                    "ctx_len": ctx_len, "pos0": pos0, "n_new": n_new, "next": nxt})
        ctx_len, pos0, n_new, block_ids = nxt["ctx_len"], nxt["pos0"], nxt["n_new"], nxt["block_ids"]
    return out
