"""Seeded synthetic inputs for one block-diffusion drafting step.

This module only draws numbers and lays them out.  It holds none of the
method's arithmetic: no norm, projection, attention, convolution, top-k, path
choice or acceptance.  Both the CPU oracle (``oracle/``) and the HIP path (via
the tests and ``bench.py``) take their inputs from here, so that the two sides
see bit-identical weights, caches, hidden states and target logits.

Conventions
-----------
* Every linear weight is ``[out, in]`` row-major.
* bf16 tensors are returned as ``numpy.uint16`` arrays holding the bf16 bit
  patterns; fp32 tensors as ``numpy.float32``.
* All draws come from ``numpy.random.Generator(PCG64)`` seeded by
  ``SeedSequence(seed, spawn_key=(tensor_index, chunk_index))``.  Large tensors
  are drawn in fixed row chunks so that the values do not depend on the number
  of threads used to draw them.

Workloads (a drafter step of the DFlash family, shapes of a Qwen3-8B-sized
drafter; the values are random-init stand-ins for trained weights):

======  =====  ======  =====================  =====  =======  ============
name    dtype  batch   context rows           conv   gate     planted logits
======  =====  ======  =====================  =====  =======  ============
c1      f32    1       128                    no     no       no
c2      bf16   1       4096                   no     no       no
c3      bf16   32      U{1024..8192} seeded   no     no       yes
c4      bf16   4       32768                  no     no       no
c5      bf16   16      16384                  yes    yes      yes
======  =====  ======  =====================  =====  =======  ============
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence

import numpy as np

BLOCK = 16
TOPK = 16
PS_DIM = 256


@dataclasses.dataclass(frozen=True)
class Dims:
    """Shapes and switches of one drafter (all sizes in elements)."""

    dtype: str            # "bf16" or "f32": storage type of weights, caches, GEMM operands
    d: int                # drafter hidden width
    n_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    n_layers: int
    n_feat_layers: int    # number of sampled target layers whose hiddens are concatenated
    d_target: int         # target hidden width
    vocab: int
    ps_rank: int          # rank of the Path Selector's bilinear form
    use_conv: bool = False
    use_gate: bool = False
    rms_eps: float = 1e-6
    rope_theta: float = 1.0e6
    block: int = BLOCK
    topk: int = TOPK
    ps_dim: int = PS_DIM

    @property
    def mask_id(self) -> int:
        return self.vocab - 1

    @property
    def d_cat(self) -> int:
        return self.n_feat_layers * self.d_target

    @property
    def group(self) -> int:
        return self.n_heads // self.n_kv_heads


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dims: Dims
    batch: int
    ctx_lens: tuple          # per sequence context rows already injected
    planted: bool            # +4 on a seeded random token per target-logit row
    seed: int
    description: str = ""

    @property
    def cap(self) -> int:
        """KV-cache rows per sequence: a multiple of 32 with room for one more block."""
        m = max(self.ctx_lens) if self.ctx_lens else 0
        return ((m + BLOCK + 31) // 32) * 32


QWEN3_8B_DRAFTER = dict(d=4096, n_heads=32, n_kv_heads=8, head_dim=128, d_ffn=12288,
                        n_layers=5, n_feat_layers=5, d_target=4096, vocab=151936)


def _c3_ctx(seed: int, batch: int) -> tuple:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(9000,))))
    return tuple(int(v) for v in rng.integers(1024, 8192, size=batch, endpoint=True))


def workload(name: str, seed: Optional[int] = None) -> Workload:
    """The five named workloads (c1..c5) plus small test variants (t_*)."""
    if name == "c1":
        dims = Dims("f32", d=256, n_heads=4, n_kv_heads=4, head_dim=64, d_ffn=1024, n_layers=1,
                    n_feat_layers=2, d_target=256, vocab=1024, ps_rank=16)
        return Workload("c1", dims, 1, (128,), False, 1 if seed is None else seed,
                        "tiny drafter step, fp32: batch 1, context 128")
    if name == "c2":
        dims = Dims("bf16", ps_rank=64, **QWEN3_8B_DRAFTER)
        return Workload("c2", dims, 1, (4096,), False, 2 if seed is None else seed,
                        "Qwen3-8B-shaped drafter step, bf16: batch 1, context 4096")
    if name == "c3":
        dims = Dims("bf16", ps_rank=64, **QWEN3_8B_DRAFTER)
        s = 3 if seed is None else seed
        return Workload("c3", dims, 32, _c3_ctx(s, 32), True, s,
                        "batched drafting, bf16: batch 32, ragged context U{1024..8192}")
    if name == "c4":
        dims = Dims("bf16", ps_rank=64, **QWEN3_8B_DRAFTER)
        return Workload("c4", dims, 4, (32768,) * 4, False, 4 if seed is None else seed,
                        "long-CoT drafting, bf16: batch 4, context 32768")
    if name == "c5":
        dims = Dims("bf16", ps_rank=64, use_conv=True, use_gate=True, **QWEN3_8B_DRAFTER)
        return Workload("c5", dims, 16, (16384,) * 16, True, 5 if seed is None else seed,
                        "full DFlash 2 step, bf16: batch 16, context 16384, conv + gate")
    # Small variants the oracle finishes in seconds; they span several tiles and
    # ragged tails (vocab not a multiple of 128, context not a multiple of 32).
    if name == "t_small":
        dims = Dims("bf16", d=512, n_heads=8, n_kv_heads=2, head_dim=64, d_ffn=1024, n_layers=2,
                    n_feat_layers=3, d_target=256, vocab=3008, ps_rank=16)
        return Workload(name, dims, 3, (37, 300, 0), True, 11 if seed is None else seed,
                        "small bf16 drafter, ragged contexts incl. empty")
    if name == "t_conv":
        dims = Dims("bf16", d=512, n_heads=8, n_kv_heads=2, head_dim=64, d_ffn=1024, n_layers=2,
                    n_feat_layers=3, d_target=256, vocab=3008, ps_rank=16, use_conv=True, use_gate=True)
        return Workload(name, dims, 2, (129, 64), True, 12 if seed is None else seed,
                        "small bf16 drafter with dynamic short conv and context gate")
    if name == "t_hd128":
        dims = Dims("bf16", d=512, n_heads=8, n_kv_heads=2, head_dim=128, d_ffn=768, n_layers=1,
                    n_feat_layers=2, d_target=512, vocab=2064, ps_rank=32, use_gate=True)
        return Workload(name, dims, 2, (1000, 333), True, 13 if seed is None else seed,
                        "small bf16 drafter with 128-wide heads, GQA group 4")
    if name == "t_f32":
        dims = Dims("f32", d=256, n_heads=4, n_kv_heads=2, head_dim=64, d_ffn=512, n_layers=2,
                    n_feat_layers=2, d_target=256, vocab=1040, ps_rank=16, use_conv=True, use_gate=True)
        return Workload(name, dims, 2, (70, 5), False, 14 if seed is None else seed,
                        "small fp32 drafter with conv and gate")
    if name == "t_batch":
        dims = Dims("bf16", d=256, n_heads=4, n_kv_heads=1, head_dim=64, d_ffn=512, n_layers=1,
                    n_feat_layers=2, d_target=256, vocab=1024, ps_rank=16)
        s = 15 if seed is None else seed
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(s, spawn_key=(9001,))))
        ctx = tuple(int(v) for v in rng.integers(0, 200, size=12, endpoint=True))
        return Workload(name, dims, 12, ctx, True, s, "bf16 batch 12 (M=192 rows), ragged contexts")
    raise KeyError(name)


WORKLOADS = ("c1", "c2", "c3", "c4", "c5")
TEST_WORKLOADS = ("t_small", "t_conv", "t_hd128", "t_f32", "t_batch")


# --------------------------------------------------------------------------------------
# drawing
# --------------------------------------------------------------------------------------

def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return the bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    nan = np.isnan(x)
    out = r.astype(np.uint16)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


_POOL_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def normal(shape: Sequence[int], std: float, seed: int, key: int, dtype: str, mean: float = 0.0) -> np.ndarray:
    """N(mean, std^2) draws of ``shape`` in ``dtype`` ("bf16" -> uint16 bits, "f32")."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    cols = shape[-1] if shape else 1
    rows = n // max(cols, 1)
    chunk_rows = max(1, (1 << 21) // max(cols, 1))
    n_chunks = max(1, (rows + chunk_rows - 1) // chunk_rows)
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)

    def one(c: int) -> None:
        r0, r1 = c * chunk_rows, min(rows, (c + 1) * chunk_rows)
        v = _rng(seed, key, c).standard_normal((r1 - r0) * cols, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        if mean != 0.0:
            v += np.float32(mean)
        out[r0 * cols:r1 * cols] = f32_to_bf16_bits(v) if dtype == "bf16" else v

    if n_chunks == 1:
        one(0)
    else:
        with ThreadPoolExecutor(_POOL_THREADS) as ex:
            list(ex.map(one, range(n_chunks)))
    return out.reshape(shape)


def const(shape: Sequence[int], value: float, dtype: str) -> np.ndarray:
    v = np.full(tuple(shape), value, dtype=np.float32)
    return f32_to_bf16_bits(v) if dtype == "bf16" else v


# --------------------------------------------------------------------------------------
# weights
# --------------------------------------------------------------------------------------

LAYER_KEYS = ("w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down", "g_attn", "g_ffn")
CONV_SITES = 4


def weight_shapes(dims: Dims) -> Dict[str, tuple]:
    """Name -> shape of every weight tensor (per-layer ones carry an ``l{i}.`` prefix)."""
    d, hd = dims.d, dims.head_dim
    s: Dict[str, tuple] = {
        "embed": (dims.vocab, d),
        "lm_head": (dims.vocab, d),
        "w_fc": (d, dims.d_cat),
        "g_fc": (d,),
        "g_final": (d,),
        "ps_left": (dims.ps_dim, d),
        "ps_right": (dims.ps_dim, d),
        "ps_gate": (dims.ps_dim, d),
        "ps_u": (dims.ps_rank, dims.ps_dim),
        "ps_v": (dims.ps_rank, dims.ps_dim),
    }
    for i in range(dims.n_layers):
        p = f"l{i}."
        s[p + "w_q"] = (dims.n_heads * hd, d)
        s[p + "w_k"] = (dims.n_kv_heads * hd, d)
        s[p + "w_v"] = (dims.n_kv_heads * hd, d)
        s[p + "w_o"] = (d, dims.n_heads * hd)
        s[p + "w_gate"] = (dims.d_ffn, d)
        s[p + "w_up"] = (dims.d_ffn, d)
        s[p + "w_down"] = (d, dims.d_ffn)
        s[p + "g_attn"] = (d,)
        s[p + "g_ffn"] = (d,)
        if dims.use_conv:
            for c in range(CONV_SITES):
                s[p + f"conv{c}.gen"] = (2 * (d // 16), d)
                s[p + f"conv{c}.w0"] = (d,)
                s[p + f"conv{c}.w1"] = (d,)
    return s


def make_weights(dims: Dims, seed: int, ps_scale: str = "config", conv_scale: str = "config",
                 zero: Sequence[str] = (), names: Optional[Sequence[str]] = None) -> Dict[str, np.ndarray]:
    """Random-init drafter weights.

    Matrices and conv taps are N(0, 0.02^2); RMSNorm gains are 1.0.
    ``ps_scale="stress"`` draws the Path Selector at a scale where its pair
    scores are of the order of the logit gaps (at N(0, 0.02^2) they are ~1e-4
    and the chosen path is always the top-1 candidate, which tests nothing).
    ``conv_scale="stress"`` / ``"mild"`` draw the conv taps and their content-dependent
    corrections at O(0.2) / O(0.05).  At the config scale the static taps are ~0.02 but the
    corrections of a unit-RMS row are ~N(0, 0.02^2 d) -- O(1.3) at d = 4096 -- which makes
    a 20-site drafter ill-conditioned (see the design notes); "mild" keeps it well
    conditioned while still exercising every term.
    Names listed in ``zero`` are returned as all-zero tensors.  ``names`` restricts the
    draw to those tensors (each tensor's values do not depend on the others).
    """
    shapes = weight_shapes(dims)
    out: Dict[str, np.ndarray] = {}
    d = dims.d
    for idx, (name, shp) in enumerate(sorted(shapes.items())):
        if names is not None and name not in names:
            continue
        base = name.split(".")[-1]
        if name in zero:
            out[name] = const(shp, 0.0, dims.dtype)
            continue
        if base.startswith("g_"):
            out[name] = const(shp, 1.0, dims.dtype)
            continue
        std = 0.02
        if ps_scale == "stress":
            if name in ("ps_left", "ps_right"):
                std = 1.0 / (0.02 * np.sqrt(d))
            elif name in ("ps_u", "ps_v"):
                std = dims.ps_rank ** -0.25 / np.sqrt(dims.ps_dim)
            elif name == "ps_gate":
                std = 1.0 / np.sqrt(d)
        if conv_scale in ("stress", "mild") and base == "gen":
            # corrections ~N(0, s^2) on unit-RMS rows: s = 0.2 (stress) or 0.05 (mild)
            std = (0.2 if conv_scale == "stress" else 0.05) / np.sqrt(d)
        if conv_scale in ("stress", "mild") and base in ("w0", "w1"):
            std = 0.2 if conv_scale == "stress" else 0.05
        out[name] = normal(shp, std, seed, 100 + idx, dims.dtype)
    return out


def make_cal_weights(dims: Dims, seed: int, cal_dim: int, std: float = 0.02) -> Dict[str, np.ndarray]:
    """Weights of the bonus-calibration MLP: ``cal_w1 [cal_dim, 2d]``, ``cal_w2 [V, cal_dim]``,
    N(0, std^2) in the storage type (drawn apart from the drafter's own weights)."""
    return {"cal_w1": normal((cal_dim, 2 * dims.d), std, seed, 9001, dims.dtype),
            "cal_w2": normal((dims.vocab, cal_dim), std, seed, 9002, dims.dtype)}


# --------------------------------------------------------------------------------------
# activations, caches, ids, logits
# --------------------------------------------------------------------------------------

def make_hidden(dims: Dims, n_rows: int, seed: int, key: int = 0) -> np.ndarray:
    """Concatenated target hidden states ``[n_rows, n_feat_layers * d_target]``, N(0,1)."""
    return normal((n_rows, dims.d_cat), 1.0, seed, 5000 + key, dims.dtype)


def make_cache(dims: Dims, ctx_lens: Sequence[int], cap: int, seed: int, std: float = 1.0,
               poison: bool = False) -> tuple:
    """A KV cache filled as if ``ctx_lens[b]`` rows had been injected.

    Returns ``(K, V)``, each ``[n_layers, batch, n_kv_heads, cap, head_dim]`` in the
    logical (row-major, value-per-position) layout.  Rows at or beyond
    ``ctx_lens[b]`` are zero, or NaN when ``poison`` is set.
    """
    B = len(ctx_lens)
    shp = (dims.n_layers, B, dims.n_kv_heads, cap, dims.head_dim)
    dt = np.uint16 if dims.dtype == "bf16" else np.float32
    K = np.zeros(shp, dtype=dt)
    V = np.zeros(shp, dtype=dt)
    fill = (np.uint16(0x7FC0) if dims.dtype == "bf16" else np.float32(np.nan)) if poison else 0
    for l in range(dims.n_layers):
        for b, n in enumerate(ctx_lens):
            kk = normal((dims.n_kv_heads, n, dims.head_dim), std, seed, 7000 + 2 * (l * 1024 + b), dims.dtype)
            vv = normal((dims.n_kv_heads, n, dims.head_dim), std, seed, 7001 + 2 * (l * 1024 + b), dims.dtype)
            K[l, b, :, :n] = kk
            V[l, b, :, :n] = vv
            K[l, b, :, n:] = fill
            V[l, b, :, n:] = fill
    return K, V


def make_block_ids(dims: Dims, batch: int, seed: int, n_fixed: int = 1) -> np.ndarray:
    """``[batch, 16]`` int32: row 0 the anchor (uniform in [0, V-1)) when ``n_fixed`` is 1,
    every other row the mask token ``V-1``."""
    ids = np.full((batch, dims.block), dims.mask_id, dtype=np.int32)
    if n_fixed:
        ids[:, 0] = _rng(seed, 6000).integers(0, dims.vocab - 1, size=batch)
    return ids


def make_target_logits(dims: Dims, batch: int, n_draft: int, seed: int, planted: str = "none",
                       draft: Optional[np.ndarray] = None, boost: float = 4.0) -> np.ndarray:
    """Target logits ``[batch, n_draft + 1, vocab]``, N(0,1) in the workload dtype.

    planted = "none"   : plain N(0,1).
              "random" : +``boost`` on one uniform random token per row.
              "prefix" : for sequence b a seeded A_b in [0, n_draft]; rows i < A_b get the
                         boost on ``draft[b, i]``, later rows on a random token (coverage of
                         every accept length; the acceptance itself is still decided by argmax).
    The boost is added in float32 before rounding to the storage type.
    """
    R = n_draft + 1
    T = _rng(seed, 8000).standard_normal((batch, R, dims.vocab), dtype=np.float32)
    if planted != "none":
        rng = _rng(seed, 8001)
        tok = rng.integers(0, dims.vocab - 1, size=(batch, R))
        if planted == "prefix":
            assert draft is not None
            A = rng.integers(0, n_draft, size=batch, endpoint=True)
            for b in range(batch):
                tok[b, :A[b]] = draft[b, :A[b]]
        bi = np.arange(batch)[:, None]
        ri = np.arange(R)[None, :]
        T[bi, ri, tok] += np.float32(boost)
    return f32_to_bf16_bits(T) if dims.dtype == "bf16" else T


def make_candidates(dims: Dims, batch: int, seed: int, logit_std: float = 1.0) -> tuple:
    """Stand-alone Path Selector inputs: distinct candidate ids per row, logits sorted
    descending, and a final hidden state ``[batch, 16, d]`` float32 with unit-RMS rows."""
    rng = _rng(seed, 8100)
    K = dims.topk
    ids = np.empty((batch, dims.block, K), dtype=np.int32)
    for b in range(batch):
        for i in range(dims.block):
            ids[b, i] = rng.choice(dims.vocab - 1, size=K, replace=False)
    lg = np.sort(rng.standard_normal((batch, dims.block, K)).astype(np.float32) * np.float32(logit_std), axis=-1)[..., ::-1]
    xh = rng.standard_normal((batch, dims.block, dims.d)).astype(np.float32)
    return ids, np.ascontiguousarray(lg), xh


def make_prefill_positions(ctx_lens: Sequence[int]) -> tuple:
    """Row layout for injecting the whole context: ``row_off [B+1]``, ``pos0 [B]``, ``n_new [B]``."""
    n = np.asarray(ctx_lens, dtype=np.int32)
    row_off = np.zeros(len(n) + 1, dtype=np.int32)
    row_off[1:] = np.cumsum(n)
    return row_off, np.zeros(len(n), dtype=np.int32), n.copy()
