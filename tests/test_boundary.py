"""The C-ABI library on the CPU: it loads, exports every declared symbol, and rejects bad
arguments before anything reaches the GPU (no compute calls are made here)."""
import ctypes
import os
import re
import sys

import pytest

import block_diffusion_drafter_feature_amd as D
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash.h")
FAKE = 0x10000          # a non-null pointer value; the rejected calls never dereference it


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(dflash_\w+)\s*\(", txt, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) == 21
    lib = ctypes.CDLL(D.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(D.EXPORTED)


def test_status_strings():
    assert D.status_string(0) == "ok"
    assert "workspace" in D.status_string(D.DFLASH_E_WORKSPACE)
    assert D.status_string(12345) == "unknown status"


@pytest.mark.parametrize("name", synth.WORKLOADS + synth.TEST_WORKLOADS)
def test_named_configs_are_supported(name):
    cfg = D.make_config(synth.workload(name).dims)
    assert D.dflash_check_config(cfg) == D.DFLASH_OK
    assert D.dflash_draft_workspace_bytes(cfg, 4, 1024) > 0
    assert D.dflash_inject_workspace_bytes(cfg, 16) > 0
    assert D.dflash_path_workspace_bytes(cfg, 4) > 0


def test_bad_configs_rejected():
    base = synth.workload("t_small").dims
    def with_(**kw):
        c = D.make_config(base)
        for k, v in kw.items():
            setattr(c, k, v)
        return D.dflash_check_config(c)
    assert with_(dtype=7) == D.DFLASH_E_INVAL
    assert with_(d_model=0) == D.DFLASH_E_INVAL
    assert with_(head_dim=96) == D.DFLASH_E_UNSUPPORTED
    assert with_(n_heads=6, n_kv_heads=4) == D.DFLASH_E_UNSUPPORTED
    assert with_(n_heads=16, n_kv_heads=2) == D.DFLASH_E_UNSUPPORTED     # GQA group 8
    assert with_(vocab=1000) == D.DFLASH_E_UNSUPPORTED
    assert with_(n_layers=17) == D.DFLASH_E_UNSUPPORTED
    assert with_(d_model=100) == D.DFLASH_E_UNSUPPORTED
    assert with_(use_conv=2) == D.DFLASH_E_INVAL
    assert D.dflash_draft_workspace_bytes(D.make_config(base), 0, 64) == 0
    assert D.dflash_verify_workspace_bytes(1, 65, 100) == 0


def _fake_structs(dims, batch=2, cap=64):
    cfg = D.make_config(dims)
    w = D.dflash_weights()
    for k in ("embed", "lm_head", "w_fc", "g_fc", "g_final", "ps_left", "ps_right", "ps_gate", "ps_u", "ps_v"):
        setattr(w, k, FAKE)
    for l in range(dims.n_layers):
        L = w.layers[l]
        for k in ("w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down", "g_attn", "g_ffn"):
            setattr(L, k, FAKE)
        for s in range(4):
            L.conv_gen[s] = L.conv_w0[s] = L.conv_w1[s] = FAKE
    kv = D.dflash_kv(batch=batch, cap=cap)
    for l in range(dims.n_layers):
        kv.k[l] = kv.vt[l] = FAKE
    return cfg, w, kv


def _status(fn, *args):
    with pytest.raises(D.DflashError) as e:
        fn(*args)
    return e.value.status


def test_calls_validate_before_launch():
    dims = synth.workload("t_conv").dims
    cfg, w, kv = _fake_structs(dims)
    ws_d = D.dflash_draft_workspace_bytes(cfg, 2, 64)
    ws_i = D.dflash_inject_workspace_bytes(cfg, 8)
    ws_p = D.dflash_path_workspace_bytes(cfg, 2)
    S = 1  # any stream value: nothing is enqueued on the error paths
    # draft
    assert _status(D.dflash_draft_block, cfg, w, kv, FAKE, FAKE, 2, FAKE, FAKE, FAKE, None, FAKE, ws_d - 1, None, S) == D.DFLASH_E_WORKSPACE
    assert _status(D.dflash_draft_block, cfg, w, kv, None, FAKE, 2, FAKE, FAKE, FAKE, None, FAKE, ws_d, None, S) == D.DFLASH_E_INVAL
    assert _status(D.dflash_draft_block, cfg, w, kv, FAKE, FAKE, 3, FAKE, FAKE, FAKE, None, FAKE, ws_d * 2, None, S) == D.DFLASH_E_CAPACITY
    w.layers[1].conv_w1[3] = None
    assert _status(D.dflash_draft_block, cfg, w, kv, FAKE, FAKE, 2, FAKE, FAKE, FAKE, None, FAKE, ws_d, None, S) == D.DFLASH_E_INVAL
    w.layers[1].conv_w1[3] = FAKE
    kv.cap = 48
    assert _status(D.dflash_draft_block, cfg, w, kv, FAKE, FAKE, 2, FAKE, FAKE, FAKE, None, FAKE, ws_d, None, S) == D.DFLASH_E_UNSUPPORTED
    kv.cap = 64
    # inject
    assert _status(D.dflash_inject_context, cfg, w, kv, FAKE, 8, FAKE, FAKE, FAKE, 2, FAKE, ws_i - 1, None, S) == D.DFLASH_E_WORKSPACE
    assert _status(D.dflash_inject_context, cfg, w, kv, FAKE, 0, FAKE, FAKE, FAKE, 2, FAKE, ws_i, None, S) == D.DFLASH_E_INVAL
    assert _status(D.dflash_inject_context, cfg, w, kv, None, 8, FAKE, FAKE, FAKE, 2, FAKE, ws_i, None, S) == D.DFLASH_E_INVAL
    # path
    assert _status(D.dflash_select_path, cfg, w, FAKE, FAKE, FAKE, FAKE, 2, 0, 2, FAKE, FAKE, None, FAKE, ws_p, S) == D.DFLASH_E_INVAL
    assert _status(D.dflash_select_path, cfg, w, FAKE, FAKE, FAKE, FAKE, 1, 5, 2, FAKE, FAKE, None, FAKE, ws_p, S) == D.DFLASH_E_INVAL
    assert _status(D.dflash_select_path, cfg, w, FAKE, FAKE, None, FAKE, 1, 0, 2, FAKE, FAKE, None, FAKE, ws_p, S) == D.DFLASH_E_INVAL
    assert _status(D.dflash_select_path, cfg, w, FAKE, FAKE, FAKE, FAKE, 1, 0, 2, FAKE, FAKE, None, FAKE, ws_p - 1, S) == D.DFLASH_E_WORKSPACE
    # verify
    ws_v = D.dflash_verify_workspace_bytes(2, 15, 1024)
    assert _status(D.dflash_verify, FAKE, FAKE, D.DFLASH_BF16, 2, 65, 1024, FAKE, FAKE, FAKE, ws_v, S) == D.DFLASH_E_UNSUPPORTED
    assert _status(D.dflash_verify, FAKE, FAKE, 9, 2, 15, 1024, FAKE, FAKE, FAKE, ws_v, S) == D.DFLASH_E_INVAL
    assert _status(D.dflash_verify, FAKE, FAKE, D.DFLASH_BF16, 2, 15, 1024, FAKE, FAKE, FAKE, ws_v - 1, S) == D.DFLASH_E_WORKSPACE
    assert _status(D.dflash_verify, None, FAKE, D.DFLASH_BF16, 2, 15, 1024, FAKE, FAKE, FAKE, ws_v, S) == D.DFLASH_E_INVAL


def test_kv_bytes_and_slice_bound():
    cfg = D.make_config(synth.workload("c2").dims)
    assert D.dflash_kv_bytes(cfg, 1, 4096) == 2 * 5 * 8 * 4096 * 128 * 2
    assert D.dflash_kv_bytes(cfg, 3, 64) == 3 * D.dflash_kv_bytes(cfg, 1, 64)
    assert D.dflash_kv_bytes(cfg, 1, 48) == 0            # not a multiple of 32
    assert D.dflash_kv_bytes(cfg, 0, 64) == 0
    # one (sequence, kv head) slice must stay below 2 GiB: cap * 128 * 2 B
    big = (1 << 31) // (128 * 2)
    assert D.dflash_kv_bytes(cfg, 1, big - 32) > 0
    assert D.dflash_kv_bytes(cfg, 1, big) == 0
    dims = synth.workload("c2").dims
    cfg, w, kv = _fake_structs(dims, batch=1, cap=big)
    ws_d = D.dflash_draft_workspace_bytes(cfg, 1, 64)
    assert _status(D.dflash_draft_block, cfg, w, kv, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None, FAKE, ws_d, None, 1) == D.DFLASH_E_UNSUPPORTED
    assert _status(D.dflash_inject_context, cfg, w, kv, FAKE, 8, FAKE, FAKE, FAKE, 1, FAKE, 1 << 40, None, 1) == D.DFLASH_E_UNSUPPORTED


def test_verify_noalloc_rejects_before_launch():
    S = 1
    assert _status(D.dflash_verify_noalloc, FAKE, FAKE, D.DFLASH_BF16, 0, 15, 1024, FAKE, FAKE, S) == D.DFLASH_E_INVAL
    assert _status(D.dflash_verify_noalloc, FAKE, FAKE, D.DFLASH_BF16, 2, 65, 1024, FAKE, FAKE, S) == D.DFLASH_E_UNSUPPORTED
    assert _status(D.dflash_verify_noalloc, FAKE, FAKE, 9, 2, 15, 1024, FAKE, FAKE, S) == D.DFLASH_E_INVAL
    assert _status(D.dflash_verify_noalloc, None, FAKE, D.DFLASH_BF16, 2, 15, 1024, FAKE, FAKE, S) == D.DFLASH_E_INVAL
    # sizes beyond the fixed scratch are refused (no launch, no allocation)
    V = 151936
    assert D.dflash_verify_workspace_bytes(431, 15, V) <= D.DFLASH_VERIFY_NOALLOC_SCRATCH
    assert D.dflash_verify_workspace_bytes(432, 15, V) > D.DFLASH_VERIFY_NOALLOC_SCRATCH
    assert _status(D.dflash_verify_noalloc, FAKE, FAKE, D.DFLASH_BF16, 432, 15, V, FAKE, FAKE, S) == D.DFLASH_E_WORKSPACE


def test_advance_rejects_bad_arguments():
    lib = D.lib()
    f = FAKE
    assert lib.dflash_advance(None, f, 1, 0, 64, f, f, f, f, None) == D.DFLASH_E_INVAL
    assert lib.dflash_advance(f, f, 0, 0, 64, f, f, f, f, None) == D.DFLASH_E_INVAL
    assert lib.dflash_advance(f, f, 1, 0, 0, f, f, f, f, None) == D.DFLASH_E_INVAL
    assert lib.dflash_advance(f, f, 1, 0, 64, f, f, None, f, None) == D.DFLASH_E_INVAL


def test_sampling_calls_reject_bad_arguments():
    dims = synth.workload("t_conv").dims
    cfg, w, kv = _fake_structs(dims)
    ws_p = D.dflash_path_workspace_bytes(cfg, 2)
    S = 1
    sp = D.dflash_sample_path
    # (cfg, w, cand_ids, cand_logits, xhat, block_ids, n_fixed, batch, t, uniforms, idx, ids, q, ps, ws, nb)
    assert _status(sp, cfg, w, FAKE, FAKE, FAKE, FAKE, 1, 2, 0.0, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws_p, S) == D.DFLASH_E_INVAL
    assert _status(sp, cfg, w, FAKE, FAKE, FAKE, FAKE, 1, 2, -1.0, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws_p, S) == D.DFLASH_E_INVAL
    assert _status(sp, cfg, w, FAKE, FAKE, FAKE, FAKE, 1, 2, float("nan"), FAKE, FAKE, FAKE, FAKE, None, FAKE, ws_p, S) == D.DFLASH_E_INVAL
    assert _status(sp, cfg, w, FAKE, FAKE, FAKE, FAKE, 1, 2, 1.0, None, FAKE, FAKE, FAKE, None, FAKE, ws_p, S) == D.DFLASH_E_INVAL
    assert _status(sp, cfg, w, FAKE, FAKE, FAKE, FAKE, 1, 2, 1.0, FAKE, FAKE, FAKE, None, None, FAKE, ws_p, S) == D.DFLASH_E_INVAL
    assert _status(sp, cfg, w, FAKE, FAKE, FAKE, FAKE, 2, 2, 1.0, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws_p, S) == D.DFLASH_E_INVAL
    assert _status(sp, cfg, w, FAKE, FAKE, FAKE, FAKE, 1, 2, 1.0, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws_p - 1, S) == D.DFLASH_E_WORKSPACE
    vs = D.dflash_verify_sampled
    ws_v = D.dflash_verify_sampled_workspace_bytes(2, 15, 1024)
    assert ws_v > 0 and D.dflash_verify_sampled_workspace_bytes(2, 65, 1024) == 0
    assert D.dflash_verify_sampled_workspace_bytes(2, 15, 4096 * 1024 + 1) == 0
    # (draft, q_ids, stride, q_probs, T, dtype, batch, n_draft, vocab, t, u_acc, u_bonus, acc, bonus, ws, nb)
    ok = (FAKE, FAKE, 256, FAKE, FAKE, D.DFLASH_BF16, 2, 15, 1024, 1.0, FAKE, FAKE, FAKE, FAKE, FAKE, ws_v, S)

    def bad(**kw):
        names = ("draft", "q_ids", "stride", "q_probs", "T", "dtype", "batch", "n_draft", "vocab", "t", "u_acc",
                 "u_bonus", "acc", "bonus", "ws", "nb", "s")
        a = dict(zip(names, ok))
        a.update(kw)
        return _status(vs, *[a[n] for n in names])
    assert bad(t=0.0) == D.DFLASH_E_INVAL
    assert bad(t=float("inf")) == D.DFLASH_E_INVAL
    assert bad(n_draft=65) == D.DFLASH_E_UNSUPPORTED
    assert bad(vocab=4096 * 1024 + 1) == D.DFLASH_E_UNSUPPORTED
    assert bad(dtype=7) == D.DFLASH_E_INVAL
    assert bad(stride=16 * 15 - 1) == D.DFLASH_E_INVAL
    assert bad(q_ids=None) == D.DFLASH_E_INVAL
    assert bad(q_probs=None) == D.DFLASH_E_INVAL
    assert bad(u_acc=None) == D.DFLASH_E_INVAL
    assert bad(u_bonus=None) == D.DFLASH_E_INVAL
    assert bad(nb=ws_v - 1) == D.DFLASH_E_WORKSPACE
    assert bad(batch=0) == D.DFLASH_E_INVAL


def test_fp8_storage_arguments():
    cfg = D.make_config(synth.workload("t_f32").dims, fp8=True)
    assert D.dflash_check_config(cfg) == D.DFLASH_E_UNSUPPORTED
    cfg = D.make_config(synth.workload("t_small").dims, fp8=True)
    assert D.dflash_check_config(cfg) == D.DFLASH_OK
    cfg.weight_format = 2
    assert D.dflash_check_config(cfg) == D.DFLASH_E_INVAL
    q = D.dflash_quantize_fp8
    assert _status(q, FAKE, 4, 100, FAKE, 1) == D.DFLASH_E_INVAL       # cols not a multiple of 64
    assert _status(q, FAKE, 0, 64, FAKE, 1) == D.DFLASH_E_INVAL
    assert _status(q, None, 4, 64, FAKE, 1) == D.DFLASH_E_INVAL
    assert _status(q, FAKE, 4, 64, FAKE + 8, 1) == D.DFLASH_E_INVAL    # output not 16-byte aligned


def test_block_size_arguments():
    dims = synth.workload("t_small").dims
    cfg = D.make_config(dims, block_size=5)
    assert cfg.block_size == 5 and D.dflash_check_config(cfg) == D.DFLASH_OK
    assert D.make_config(dims).block_size == 16
    for bad in (0, 17, -1):
        cfg.block_size = bad
        assert D.dflash_check_config(cfg) == D.DFLASH_E_INVAL
    # a one-row block with an anchor leaves nothing to choose
    cfg, w, kv = _fake_structs(dims)
    cfg.block_size = 1
    ws_p = D.dflash_path_workspace_bytes(cfg, 2)
    assert _status(D.dflash_select_path, cfg, w, FAKE, FAKE, FAKE, FAKE, 1, 0, 2, FAKE, FAKE, None, FAKE, ws_p, 1) == D.DFLASH_E_INVAL


def test_calibrate_arguments():
    dims = synth.workload("t_small").dims
    cfg, w, kv = _fake_structs(dims)
    assert D.dflash_calibrate_workspace_bytes(cfg, 2) == 0          # no calibration MLP configured
    assert _status(D.dflash_calibrate, cfg, w, FAKE, FAKE, 2, FAKE, FAKE, FAKE, FAKE, 1 << 20, 1) == D.DFLASH_E_INVAL
    cfg.cal_dim = 100
    assert D.dflash_check_config(cfg) == D.DFLASH_E_INVAL
    cfg.cal_dim = 64
    nb = D.dflash_calibrate_workspace_bytes(cfg, 2)
    assert nb > 0
    assert _status(D.dflash_calibrate, cfg, w, FAKE, FAKE, 2, FAKE, FAKE, FAKE, FAKE, nb, 1) == D.DFLASH_E_INVAL
    w.cal_w1 = w.cal_w2 = FAKE
    assert _status(D.dflash_calibrate, cfg, w, FAKE, FAKE, 2, FAKE, FAKE, FAKE, FAKE, nb - 1, 1) == D.DFLASH_E_WORKSPACE
    assert _status(D.dflash_calibrate, cfg, w, FAKE, None, 2, FAKE, FAKE, FAKE, FAKE, nb, 1) == D.DFLASH_E_INVAL


def test_bench_refuses_more_than_one_gpu():
    """The benchmark measures one GPU: any other --gpus value ends with a message and a nonzero
    status before anything touches a device."""
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for n in (2, 8):
        p = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", str(n)],
                           capture_output=True, text=True, timeout=120, cwd=root)
        assert p.returncode != 0, n
        assert "one GPU only" in p.stderr and p.stdout.strip() == "", (n, p.stderr, p.stdout)
