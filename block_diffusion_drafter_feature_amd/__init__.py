"""Python binding of the drafting-step library (``libdflash.so``, C ABI in ``include/dflash.h``).

Thin by design: the functions below carry the C calls' names and do argument
marshalling only (tensors -> device pointers, the current torch stream -> a HIP
stream, status codes -> exceptions).  Every step of the computation runs in the
library's HIP kernels.  PyTorch provides device memory and streams.

The library must have been built (``python -m block_diffusion_drafter_feature_amd.build``
or ``__graft_entry__.build()``); importing this package does not build it and
there is no fallback: without the library every call raises.

Helpers ``Drafter`` (device weights + the config/weights structs), ``KVCache`` and
``Workspace`` only allocate and lay out memory.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdflash.so")

DFLASH_OK = 0
DFLASH_E_INVAL = -1
DFLASH_E_UNSUPPORTED = -2
DFLASH_E_WORKSPACE = -3
DFLASH_E_CAPACITY = -4
DFLASH_E_HIP = -5
DFLASH_WEIGHTS_DTYPE = 0
DFLASH_WEIGHTS_FP8 = 1
DFLASH_F32 = 0
DFLASH_BF16 = 1
DFLASH_PATH_GREEDY = 0
DFLASH_PATH_EXACT = 1
MAX_LAYERS = 16
CONV_SITES = 4
BLOCK = 16
PROBES = ("lm_head", "topk", "attn", "qkv", "o", "gate_up", "down", "inject_fc", "inject_kv", "conv_pre",
          "conv_post")
N_PROBES = len(PROBES)

EXPORTED = (
    "dflash_inject_context", "dflash_draft_block", "dflash_select_path", "dflash_verify", "dflash_advance",
    "dflash_sample_path", "dflash_verify_sampled", "dflash_quantize_fp8", "dflash_calibrate",
    "dflash_calibrate_workspace_bytes", "dflash_path_table_bytes", "dflash_build_path_table",
    "dflash_inject_workspace_bytes", "dflash_draft_workspace_bytes", "dflash_path_workspace_bytes",
    "dflash_verify_workspace_bytes", "dflash_verify_sampled_workspace_bytes", "dflash_check_config",
    "dflash_status_string", "dflash_kv_bytes", "dflash_verify_noalloc",
)


class DflashError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")
        self.status = status


# ------------------------------------------------------------------ C structs

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32


class dflash_config(ctypes.Structure):
    _fields_ = [("dtype", _i32), ("d_model", _i32), ("n_heads", _i32), ("n_kv_heads", _i32),
                ("head_dim", _i32), ("d_ffn", _i32), ("n_layers", _i32), ("n_feat_layers", _i32),
                ("d_target", _i32), ("vocab", _i32), ("ps_dim", _i32), ("ps_rank", _i32),
                ("use_conv", _i32), ("use_gate", _i32), ("rms_eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float), ("weight_format", _i32), ("block_size", _i32),
                ("cal_dim", _i32)]


class dflash_layer_weights(ctypes.Structure):
    _fields_ = [("w_q", _vp), ("w_k", _vp), ("w_v", _vp), ("w_o", _vp), ("w_gate", _vp), ("w_up", _vp),
                ("w_down", _vp), ("g_attn", _vp), ("g_ffn", _vp), ("conv_gen", _vp * CONV_SITES),
                ("conv_w0", _vp * CONV_SITES), ("conv_w1", _vp * CONV_SITES)]


class dflash_weights(ctypes.Structure):
    _fields_ = [("embed", _vp), ("lm_head", _vp), ("w_fc", _vp), ("g_fc", _vp), ("g_final", _vp),
                ("ps_left", _vp), ("ps_right", _vp), ("ps_gate", _vp), ("ps_u", _vp), ("ps_v", _vp),
                ("layers", dflash_layer_weights * MAX_LAYERS), ("cal_w1", _vp), ("cal_w2", _vp),
                ("ps_table", _vp)]


class dflash_probes(ctypes.Structure):
    _fields_ = [("begin", _vp * N_PROBES), ("end", _vp * N_PROBES)]


class dflash_kv(ctypes.Structure):
    _fields_ = [("k", _vp * MAX_LAYERS), ("vt", _vp * MAX_LAYERS), ("batch", _i32), ("cap", _i32)]


# ------------------------------------------------------------------ library loading

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_diffusion_drafter_feature_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, PC = ctypes.POINTER, ctypes.c_size_t
        cfgp, wp, kvp, pp = P(dflash_config), P(dflash_weights), P(dflash_kv), P(dflash_probes)
        sig = {
            "dflash_inject_context": ([cfgp, wp, kvp, _vp, _i32, _vp, _vp, _vp, _i32, _vp, PC, pp, _vp], ctypes.c_int),
            "dflash_draft_block": ([cfgp, wp, kvp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, PC, pp, _vp],
                                   ctypes.c_int),
            "dflash_select_path": ([cfgp, wp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, PC, _vp],
                                   ctypes.c_int),
            "dflash_verify": ([_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, PC, _vp], ctypes.c_int),
            "dflash_advance": ([_vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
            "dflash_sample_path": ([cfgp, wp, _vp, _vp, _vp, _vp, _i32, _i32, ctypes.c_float, _vp, _vp, _vp, _vp,
                                    _vp, _vp, PC, _vp], ctypes.c_int),
            "dflash_verify_sampled": ([_vp, _vp, ctypes.c_int64, _vp, _vp, _i32, _i32, _i32, _i32, ctypes.c_float,
                                       _vp, _vp, _vp, _vp, _vp, PC, _vp], ctypes.c_int),
            "dflash_verify_sampled_workspace_bytes": ([_i32, _i32, _i32], PC),
            "dflash_quantize_fp8": ([_vp, _i32, _i32, _vp, _vp], ctypes.c_int),
            "dflash_calibrate": ([cfgp, wp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, PC, _vp], ctypes.c_int),
            "dflash_calibrate_workspace_bytes": ([cfgp, _i32], PC),
            "dflash_path_table_bytes": ([cfgp], PC),
            "dflash_build_path_table": ([cfgp, wp, _vp, _vp], ctypes.c_int),
            "dflash_inject_workspace_bytes": ([cfgp, _i32], PC),
            "dflash_draft_workspace_bytes": ([cfgp, _i32, _i32], PC),
            "dflash_path_workspace_bytes": ([cfgp, _i32], PC),
            "dflash_verify_workspace_bytes": ([_i32, _i32, _i32], PC),
            "dflash_check_config": ([cfgp], ctypes.c_int),
            "dflash_kv_bytes": ([cfgp, _i32, _i32], PC),
            "dflash_verify_noalloc": ([_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp], ctypes.c_int),
            "dflash_status_string": ([ctypes.c_int], ctypes.c_char_p),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _ptr(x) -> Optional[int]:
    """Device pointer of a tensor (or an int / None passed through)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int) -> None:
    if status != DFLASH_OK:
        raise DflashError(fn, status)


def status_string(status: int) -> str:
    return lib().dflash_status_string(status).decode()


# ------------------------------------------------------------------ the calls (same names as the C ABI)

def dflash_check_config(cfg: dflash_config) -> int:
    return lib().dflash_check_config(ctypes.byref(cfg))


def dflash_inject_workspace_bytes(cfg: dflash_config, n_rows: int) -> int:
    return lib().dflash_inject_workspace_bytes(ctypes.byref(cfg), n_rows)


def dflash_draft_workspace_bytes(cfg: dflash_config, batch: int, cap: int) -> int:
    return lib().dflash_draft_workspace_bytes(ctypes.byref(cfg), batch, cap)


def dflash_kv_bytes(cfg: dflash_config, batch: int, cap: int) -> int:
    return lib().dflash_kv_bytes(ctypes.byref(cfg), batch, cap)


def dflash_path_workspace_bytes(cfg: dflash_config, batch: int) -> int:
    return lib().dflash_path_workspace_bytes(ctypes.byref(cfg), batch)


def dflash_verify_workspace_bytes(batch: int, n_draft: int, vocab: int) -> int:
    return lib().dflash_verify_workspace_bytes(batch, n_draft, vocab)


def dflash_advance(accept_len, bonus, batch, mask_id, cap, ctx_len, pos0, n_new, block_ids, stream=None) -> None:
    _check("dflash_advance", lib().dflash_advance(
        _ptr(accept_len), _ptr(bonus), batch, mask_id, cap, _ptr(ctx_len), _ptr(pos0), _ptr(n_new), _ptr(block_ids),
        _stream(stream)))


def _probes(p):
    return None if p is None else ctypes.byref(p)


def dflash_inject_context(cfg, w, kv, hidden, n_rows, row_off, pos0, n_new, batch, workspace, workspace_bytes,
                          probes=None, stream=None) -> None:
    _check("dflash_inject_context", lib().dflash_inject_context(
        ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), _ptr(hidden), n_rows, _ptr(row_off), _ptr(pos0),
        _ptr(n_new), batch, _ptr(workspace), workspace_bytes, _probes(probes), _stream(stream)))


def dflash_draft_block(cfg, w, kv, ctx_len, block_ids, batch, cand_ids, cand_logits, final_hidden, logits,
                       workspace, workspace_bytes, probes=None, stream=None) -> None:
    _check("dflash_draft_block", lib().dflash_draft_block(
        ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), _ptr(ctx_len), _ptr(block_ids), batch,
        _ptr(cand_ids), _ptr(cand_logits), _ptr(final_hidden), _ptr(logits), _ptr(workspace), workspace_bytes,
        _probes(probes), _stream(stream)))


def dflash_select_path(cfg, w, cand_ids, cand_logits, final_hidden, block_ids, n_fixed, mode, batch, path_idx,
                       path_ids, pair_scores, workspace, workspace_bytes, stream=None) -> None:
    _check("dflash_select_path", lib().dflash_select_path(
        ctypes.byref(cfg), ctypes.byref(w), _ptr(cand_ids), _ptr(cand_logits), _ptr(final_hidden), _ptr(block_ids),
        n_fixed, mode, batch, _ptr(path_idx), _ptr(path_ids), _ptr(pair_scores), _ptr(workspace), workspace_bytes,
        _stream(stream)))


def dflash_sample_path(cfg, w, cand_ids, cand_logits, final_hidden, block_ids, n_fixed, batch, temperature,
                       uniforms, path_idx, path_ids, path_q, pair_scores, workspace, workspace_bytes,
                       stream=None) -> None:
    _check("dflash_sample_path", lib().dflash_sample_path(
        ctypes.byref(cfg), ctypes.byref(w), _ptr(cand_ids), _ptr(cand_logits), _ptr(final_hidden), _ptr(block_ids),
        n_fixed, batch, temperature, _ptr(uniforms), _ptr(path_idx), _ptr(path_ids), _ptr(path_q),
        _ptr(pair_scores), _ptr(workspace), workspace_bytes, _stream(stream)))


def dflash_verify_sampled_workspace_bytes(batch: int, n_draft: int, vocab: int) -> int:
    return lib().dflash_verify_sampled_workspace_bytes(batch, n_draft, vocab)


def dflash_verify_sampled(draft, q_ids, q_ids_stride, q_probs, tgt_logits, tgt_dtype, batch, n_draft, vocab,
                          temperature, u_accept, u_bonus, accept_len, bonus, workspace, workspace_bytes,
                          stream=None) -> None:
    _check("dflash_verify_sampled", lib().dflash_verify_sampled(
        _ptr(draft), _ptr(q_ids), q_ids_stride, _ptr(q_probs), _ptr(tgt_logits), tgt_dtype, batch, n_draft, vocab,
        temperature, _ptr(u_accept), _ptr(u_bonus), _ptr(accept_len), _ptr(bonus), _ptr(workspace),
        workspace_bytes, _stream(stream)))


def dflash_verify(draft, tgt_logits, tgt_dtype, batch, n_draft, vocab, accept_len, bonus, workspace,
                  workspace_bytes, stream=None) -> None:
    _check("dflash_verify", lib().dflash_verify(
        _ptr(draft), _ptr(tgt_logits), tgt_dtype, batch, n_draft, vocab, _ptr(accept_len), _ptr(bonus),
        _ptr(workspace), workspace_bytes, _stream(stream)))


DFLASH_VERIFY_NOALLOC_SCRATCH = 1 << 20


def dflash_verify_noalloc(draft, tgt_logits, tgt_dtype, batch, n_draft, vocab, accept_len, bonus,
                          stream=None) -> None:
    _check("dflash_verify_noalloc", lib().dflash_verify_noalloc(
        _ptr(draft), _ptr(tgt_logits), tgt_dtype, batch, n_draft, vocab, _ptr(accept_len), _ptr(bonus),
        _stream(stream)))


_hip = None


def hip() -> ctypes.CDLL:
    """The HIP runtime (for events the library records on the caller's stream)."""
    global _hip
    if _hip is None:
        lib()                     # the library links the runtime; load it first
        for name in ("libamdhip64.so", "libamdhip64.so.7", "libamdhip64.so.6"):
            try:
                _hip = ctypes.CDLL(name)
                break
            except OSError:
                continue
        if _hip is None:
            raise RuntimeError("HIP runtime (libamdhip64.so) not found")
        _hip.hipEventCreate.argtypes = [ctypes.POINTER(_vp)]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _vp, _vp]
        _hip.hipEventDestroy.argtypes = [_vp]
    return _hip


class Probes:
    """HIP events for the timing probes of inject/draft calls (see dflash_probes)."""

    def __init__(self, names=PROBES):
        H = hip()
        self.struct = dflash_probes()
        self.ev = {}
        for n in names:
            pair = []
            for _ in range(2):
                e = _vp()
                if H.hipEventCreate(ctypes.byref(e)) != 0:
                    raise RuntimeError("hipEventCreate failed")
                pair.append(e)
            i = PROBES.index(n)
            self.struct.begin[i] = pair[0]
            self.struct.end[i] = pair[1]
            self.ev[n] = pair

    def ms(self, name: str) -> float:
        b, e = self.ev[name]
        out = ctypes.c_float()
        st = hip().hipEventElapsedTime(ctypes.byref(out), b, e)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st}) for probe {name}")
        return float(out.value)

    def __del__(self):
        try:
            for b, e in self.ev.values():
                hip().hipEventDestroy(b)
                hip().hipEventDestroy(e)
        except Exception:
            pass


# ------------------------------------------------------------------ memory helpers (allocation / layout only)

def make_config(dims, fp8: bool = False, block_size: Optional[int] = None) -> dflash_config:
    """A ``dflash_config`` from an object with the attributes of ``synth.Dims``; ``fp8``
    selects FP8 storage of the streamed projections, ``block_size`` the rows of the drafted
    block (default: the full block of 16)."""
    return dflash_config(weight_format=DFLASH_WEIGHTS_FP8 if fp8 else DFLASH_WEIGHTS_DTYPE,
        block_size=block_size or getattr(dims, "block", BLOCK),
        dtype=DFLASH_BF16 if dims.dtype == "bf16" else DFLASH_F32, d_model=dims.d, n_heads=dims.n_heads,
        n_kv_heads=dims.n_kv_heads, head_dim=dims.head_dim, d_ffn=dims.d_ffn, n_layers=dims.n_layers,
        n_feat_layers=dims.n_feat_layers, d_target=dims.d_target, vocab=dims.vocab, ps_dim=dims.ps_dim,
        ps_rank=dims.ps_rank, use_conv=int(dims.use_conv), use_gate=int(dims.use_gate),
        rms_eps=dims.rms_eps, rope_theta=dims.rope_theta)


def torch_dtype(dims):
    import torch
    return torch.bfloat16 if dims.dtype == "bf16" else torch.float32


def to_device(arr, dims, device="cuda"):
    """Upload a stored array (bf16 bit patterns as uint16, or float32) as a device tensor."""
    import numpy as np
    import torch
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def dflash_path_table_bytes(cfg) -> int:
    return lib().dflash_path_table_bytes(ctypes.byref(cfg))


def dflash_build_path_table(cfg, w, table, stream=None) -> None:
    _check("dflash_build_path_table", lib().dflash_build_path_table(ctypes.byref(cfg), ctypes.byref(w), _ptr(table),
                                                                    _stream(stream)))


def dflash_calibrate_workspace_bytes(cfg, batch: int) -> int:
    return lib().dflash_calibrate_workspace_bytes(ctypes.byref(cfg), batch)


def dflash_calibrate(cfg, w, final_hidden, bonus, batch, logits, cand_ids, cand_logits, workspace, workspace_bytes,
                     stream=None) -> None:
    _check("dflash_calibrate", lib().dflash_calibrate(
        ctypes.byref(cfg), ctypes.byref(w), _ptr(final_hidden), _ptr(bonus), batch, _ptr(logits), _ptr(cand_ids),
        _ptr(cand_logits), _ptr(workspace), workspace_bytes, _stream(stream)))


def dflash_quantize_fp8(w, rows: int, cols: int, out, stream=None) -> None:
    _check("dflash_quantize_fp8", lib().dflash_quantize_fp8(_ptr(w), rows, cols, _ptr(out), _stream(stream)))


FP8_MATRICES = ("w_fc", "lm_head", "w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down")


class Drafter:
    """Device copies of a drafter's weights and the structs that point at them.  With
    ``fp8=True`` the streamed projections are uploaded in bf16 and turned into FP8
    storage (E4M3 rows with a float32 scale) by ``dflash_quantize_fp8``."""

    def __init__(self, dims, weights: Dict[str, "object"], device: str = "cuda", fp8: bool = False,
                 block_size: Optional[int] = None, path_table: bool = True):
        import torch
        self.dims = dims
        self.fp8 = fp8
        self.t = {}
        for k, v in weights.items():
            # device tensors are used as they are (shared), host arrays uploaded
            t = v if isinstance(v, torch.Tensor) and v.is_cuda else to_device(v, dims, device)
            if fp8 and k.split(".")[-1] in FP8_MATRICES:
                rows, cols = t.shape
                q = torch.empty(rows * (cols + 16), dtype=torch.uint8, device=device)
                dflash_quantize_fp8(t, rows, cols, q)
                torch.cuda.synchronize()
                t = q
            self.t[k] = t
        self.cfg = make_config(dims, fp8, block_size)
        st = dflash_check_config(self.cfg)
        if st != DFLASH_OK:
            raise DflashError("dflash_check_config", st)
        w = dflash_weights()
        p = lambda k: self.t[k].data_ptr() if k in self.t else None  # noqa: E731
        for k in ("embed", "lm_head", "w_fc", "g_fc", "g_final", "ps_left", "ps_right", "ps_gate", "ps_u", "ps_v",
                  "cal_w1", "cal_w2"):
            setattr(w, k, p(k))
        if "cal_w1" in self.t:
            self.cfg.cal_dim = self.t["cal_w1"].shape[0]
        for l in range(dims.n_layers):
            L = w.layers[l]
            for k in ("w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down", "g_attn", "g_ffn"):
                setattr(L, k, p(f"l{l}.{k}"))
            if dims.use_conv:
                for s in range(CONV_SITES):
                    L.conv_gen[s] = p(f"l{l}.conv{s}.gen")
                    L.conv_w0[s] = p(f"l{l}.conv{s}.w0")
                    L.conv_w1[s] = p(f"l{l}.conv{s}.w1")
        self.w = w
        self.table = None
        if path_table and all(k in self.t for k in ("embed", "ps_left", "ps_right")):
            # the Path Selector's per-token projections, built once on the device
            self.table = torch.empty(dflash_path_table_bytes(self.cfg) // 4, dtype=torch.float32, device=device)
            dflash_build_path_table(self.cfg, w, self.table)
            torch.cuda.synchronize()
            w.ps_table = self.table.data_ptr()

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.t.values())


class KVCache:
    """Per-layer key cache ``[B][Hkv][cap][hd]`` and transposed value cache ``[B][Hkv][hd][cap]``."""

    def __init__(self, dims, batch: int, cap: int, device: str = "cuda", fill: Optional[float] = 0.0):
        import torch
        if cap % 32:
            raise ValueError("cap must be a multiple of 32")
        dt = torch_dtype(dims)
        shp = (batch, dims.n_kv_heads, cap, dims.head_dim)
        shpt = (batch, dims.n_kv_heads, dims.head_dim, cap)
        if fill is None:
            self.k = [torch.empty(shp, dtype=dt, device=device) for _ in range(dims.n_layers)]
            self.vt = [torch.empty(shpt, dtype=dt, device=device) for _ in range(dims.n_layers)]
        else:
            self.k = [torch.full(shp, fill, dtype=dt, device=device) for _ in range(dims.n_layers)]
            self.vt = [torch.full(shpt, fill, dtype=dt, device=device) for _ in range(dims.n_layers)]
        self.dims, self.batch, self.cap = dims, batch, cap
        kv = dflash_kv(batch=batch, cap=cap)
        for l in range(dims.n_layers):
            kv.k[l] = self.k[l].data_ptr()
            kv.vt[l] = self.vt[l].data_ptr()
        self.kv = kv

    def load_logical(self, K, V) -> None:
        """Copy caches given as ``[L][B][Hkv][cap][hd]`` stored arrays into the device layout."""
        for l in range(self.dims.n_layers):
            self.k[l].copy_(to_device(K[l], self.dims))
            self.vt[l].copy_(to_device(V[l], self.dims).transpose(-1, -2))

    def logical(self, layer: int):
        """(K, V) of one layer as ``[B][Hkv][cap][hd]`` device tensors (V transposed back)."""
        return self.k[layer], self.vt[layer].transpose(-1, -2)

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.k + self.vt)


class Workspace:
    """A device byte buffer that grows to the largest size asked for."""

    def __init__(self, device: str = "cuda"):
        self.device = device
        self.buf = None

    def get(self, nbytes: int):
        import torch
        if nbytes <= 0:
            raise DflashError("workspace size query", DFLASH_E_INVAL)
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return self.buf
