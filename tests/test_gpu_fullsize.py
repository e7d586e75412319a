"""Parity at the full workload sizes, in the launch configuration bench.py times.

Each workload runs its whole batch on the GPU (same batch, cache capacity and
calls as the timed step); the oracle recomputes sampled sequences one by one
(sequences are independent in every call).  Caches are seeded inputs written
directly for the sampled sequences (other sequences get device noise of the same
scale), so the oracle never needs a GPU-computed value.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
import block_diffusion_drafter_feature_amd as D  # noqa: E402


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def ws(n):
    return torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")


_STATE = {}


def drafter_for(name, conv_scale, fp8=False):
    """Weights, oracle model and device drafter for a workload (shared by workloads of equal
    shape; a different conv scale redraws only the conv tensors; fp8 selects FP8 storage of
    the streamed projections on both sides)."""
    wl = synth.workload(name)
    key = (wl.dims.use_conv, wl.dims.use_gate)
    if key not in _STATE:
        _STATE.clear()
        torch.cuda.empty_cache()
        _STATE[key] = {"W": synth.make_weights(wl.dims, 77, conv_scale=conv_scale), "scale": conv_scale}
    st = _STATE[key]
    if st["scale"] != conv_scale or "dr" not in st or st.get("fp8") != fp8:
        if st["scale"] != conv_scale:
            conv = [n for n in st["W"] if ".conv" in n]
            st["W"].update(synth.make_weights(wl.dims, 77, conv_scale=conv_scale, names=conv))
            st["scale"] = conv_scale
        st.pop("dr", None)
        torch.cuda.empty_cache()
        st["m"] = oracle.Model(wl.dims, st["W"], fp8=fp8)
        st["dr"] = D.Drafter(wl.dims, st["W"], fp8=fp8)
        st["fp8"] = fp8
    return wl, (st["W"], st["m"], st["dr"])


# (workload, sampled sequences, conv scale, fp8).  Every case is held to the stated 2e-2
# except c5 at its own random-init conv scale, where the conv corrections are O(1.3) per
# channel and the computation is ill-conditioned: the oracle itself moves by 6-7e-2 under
# fp32-level noise there, so that one case (CONDITIONED) is bounded by three times that
# spread, and its top-16 is checked stage-wise only (exactly the top 16 of the device's own
# logits).  c5 also runs at a milder conv scale, held to 2e-2.  FP8 storage cases: c2 (one
# block: weight-streaming kernels) and c4 (4 blocks: the pipelined kernel at 64 rows).
CASES = [("c2", (0,), "config", False), ("c3", (0, 31), "config", False), ("c4", (3,), "config", False),
         ("c5", (0, 15), "config", False), ("c5", (15,), "mild", False), ("c2", (0,), "config", True),
         ("c4", (1,), "config", True)]
CONDITIONED = {("c5", "config", False)}


@pytest.mark.parametrize("name,sample,conv_scale,fp8", CASES)
def test_fullsize_step(name, sample, conv_scale, fp8):
    wl, (W, m, dr) = drafter_for(name, conv_scale, fp8)
    dims = wl.dims
    B, cap = wl.batch, wl.cap
    ctx = np.asarray(wl.ctx_lens, dtype=np.int32)
    say(f"fullsize {name} (conv {conv_scale}{', fp8 weights' if fp8 else ''}): batch {B}, contexts {ctx.min()}..{ctx.max()}, sampled {sample}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(123)
    cache = D.KVCache(dims, B, cap, fill=None)
    scale = 0.02 * dims.d ** 0.5
    for l in range(dims.n_layers):
        for t in (cache.k[l], cache.vt[l]):
            t.copy_((torch.randn(t.shape, generator=gen, device="cuda") * scale).to(D.torch_dtype(dims)))
    # seeded caches for the sampled sequences, as if their context had been injected
    host = {}
    for b in sample:
        K, V = synth.make_cache(dims, [int(ctx[b])], cap, 500 + b, std=scale)
        host[b] = (K, V)
        for l in range(dims.n_layers):
            cache.k[l][b].copy_(D.to_device(K[l, 0], dims))
            cache.vt[l][b].copy_(D.to_device(V[l, 0], dims).transpose(-1, -2))

    # ---- inject 16 rows per sequence at L-16..L-1 (the timed step's inject)
    new = synth.make_hidden(dims, 16 * B, 600)
    pos0 = np.maximum(ctx - 16, 0)
    n_new = np.minimum(ctx, 16)
    nb = D.dflash_inject_workspace_bytes(dr.cfg, 16 * B)
    D.dflash_inject_context(dr.cfg, dr.w, cache.kv, D.to_device(new, dims), 16 * B, i32(np.arange(B + 1) * 16),
                            i32(pos0), i32(n_new), B, ws(nb), nb)
    torch.cuda.synchronize()
    t = H.tol(dims)
    ocache = {}
    for b in sample:
        n = int(n_new[b])
        pos = pos0[b] + np.arange(n)
        _, Ko, Vo = oracle.inject_rows(m, new[16 * b:16 * b + n], pos)
        K, V = host[b]
        kc = [oracle.decode(K[l, 0], dims.dtype) for l in range(dims.n_layers)]
        vc = [oracle.decode(V[l, 0], dims.dtype) for l in range(dims.n_layers)]
        for l in range(dims.n_layers):
            Kg = cache.k[l][b].float().cpu().numpy()
            Vg = cache.vt[l][b].float().cpu().numpy()
            H.assert_close_rows(f"{name} inject K b{b} l{l}", Kg[:, pos].transpose(1, 0, 2), Ko[l], t)
            H.assert_close_rows(f"{name} inject V b{b} l{l}", Vg[:, :, pos].transpose(2, 0, 1), Vo[l], t)
            # the oracle's own cache: seeded rows with its own injected rows in place
            kc[l][:, pos] = np.transpose(Ko[l], (1, 0, 2))
            vc[l][:, pos] = np.transpose(Vo[l], (1, 0, 2))
        ocache[b] = (kc, vc)

    # ---- draft the block
    ids = synth.make_block_ids(dims, B, 700, 1)
    ci = torch.zeros((B, 16, 16), dtype=torch.int32, device="cuda")
    cl = torch.zeros((B, 16, 16), dtype=torch.float32, device="cuda")
    fh = torch.zeros((B, 16, dims.d), dtype=torch.float32, device="cuda")
    lg = torch.zeros((B, 16, dims.vocab), dtype=torch.float32, device="cuda")
    nb = D.dflash_draft_workspace_bytes(dr.cfg, B, cap)
    D.dflash_draft_block(dr.cfg, dr.w, cache.kv, i32(ctx), i32(ids), B, ci, cl, fh, lg, ws(nb), nb)
    torch.cuda.synchronize()
    ci_h, cl_h, fh_h = ci.cpu().numpy(), cl.cpu().numpy(), fh.cpu().numpy()
    # the timed launch passes no logits buffer (at one drafted block the LM head then keeps
    # its top-16 lists without writing the logits): same candidates and hidden rows, bit for bit
    ci2, cl2, fh2 = torch.zeros_like(ci), torch.zeros_like(cl), torch.zeros_like(fh)
    D.dflash_draft_block(dr.cfg, dr.w, cache.kv, i32(ctx), i32(ids), B, ci2, cl2, fh2, None, ws(nb), nb)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ci2.cpu().numpy(), ci_h)
    np.testing.assert_array_equal(cl2.cpu().numpy(), cl_h)
    np.testing.assert_array_equal(fh2.cpu().numpy(), fh_h)
    for b in sample:
        kc, vc = ocache[b]
        o = oracle.draft_block(m, kc, vc, int(ctx[b]), ids[b])
        conditioned = (name, conv_scale, fp8) in CONDITIONED
        if conditioned:
            kappa = H.conditioning(m, kc, vc, int(ctx[b]), ids[b], o)
            td = H.tol_conditioned(dims, kappa)
            say(f"  b{b}: oracle fp32-level spread {kappa:.2e} -> tolerance {td:.2e}")
        else:
            td = t
        lgb = lg[b].cpu().numpy()
        H.assert_close_rows(f"{name} logits b{b}", lgb, o["logits"], td)
        H.assert_close_rows(f"{name} final hidden b{b}", fh_h[b], o["xhat"], td)
        # stage-wise exact: the candidates are exactly the top 16 of the device's own logits
        np.testing.assert_array_equal(ci_h[b], H.exact_topk_of(lgb))
        if conditioned:
            oi, _ = oracle.topk(o["logits"], 16)
            say(f"  b{b}: logits rel err {H.rowwise_relerr(lgb, o['logits']):.2e}, top-16 ranks differing from "
                f"the oracle's (not asserted in this ill-conditioned case) {int((oi != ci_h[b]).sum())}")
        else:
            near = H.topk_with_margin(ci_h[b], o["logits"], lgb)
            say(f"  b{b}: logits rel err {H.rowwise_relerr(lgb, o['logits']):.2e}, near-tie top-16 swaps {near}")

    # ---- the step's own chain (device candidates -> path -> verify): properties only
    pidx = torch.zeros((B, 15), dtype=torch.int32, device="cuda")
    pids = torch.zeros((B, 15), dtype=torch.int32, device="cuda")
    ps = torch.zeros((B, 15, 16, 16), dtype=torch.float32, device="cuda")
    nb = D.dflash_path_workspace_bytes(dr.cfg, B)
    D.dflash_select_path(dr.cfg, dr.w, ci, cl, fh, i32(ids), 1, D.DFLASH_PATH_GREEDY, B, pidx, pids, ps, ws(nb), nb)
    T = synth.make_target_logits(dims, B, 15, 800, planted="random")
    acc = torch.zeros(B, dtype=torch.int32, device="cuda")
    bon = torch.zeros(B, dtype=torch.int32, device="cuda")
    tdt = D.DFLASH_BF16 if dims.dtype == "bf16" else D.DFLASH_F32
    nb = D.dflash_verify_workspace_bytes(B, 15, dims.vocab)
    D.dflash_verify(pids, D.to_device(T, dims), tdt, B, 15, dims.vocab, acc, bon, ws(nb), nb)
    torch.cuda.synchronize()
    pidx_h, pids_h, ps_h = pidx.cpu().numpy(), pids.cpu().numpy(), ps.cpu().numpy()
    Tf = synth.bits_to_f32(T) if dims.dtype == "bf16" else T
    for b in range(B):
        np.testing.assert_array_equal(pidx_h[b], H.walk_f32(cl_h[b, 1:], ps_h[b], True, "greedy"))
        np.testing.assert_array_equal(pids_h[b], ci_h[b, 1:][np.arange(15), pidx_h[b]])
        assert (int(acc[b]), int(bon[b])) == H.accept_of(pids_h[b], Tf[b])

    # ---- Path Selector and verification at full size on seeded inputs, against the oracle
    cids, clg, xh = synth.make_candidates(dims, B, 900)
    bids = synth.make_block_ids(dims, B, 901, 1)
    nb = D.dflash_path_workspace_bytes(dr.cfg, B)
    D.dflash_select_path(dr.cfg, dr.w, i32(cids), torch.from_numpy(clg).cuda(), torch.from_numpy(xh).cuda(),
                         i32(bids), 1, D.DFLASH_PATH_GREEDY, B, pidx, pids, ps, ws(nb), nb)
    draft = np.random.default_rng(902).integers(0, dims.vocab - 1, size=(B, 15)).astype(np.int32)
    T2 = synth.make_target_logits(dims, B, 15, 903, planted="prefix", draft=draft)
    nb = D.dflash_verify_workspace_bytes(B, 15, dims.vocab)
    D.dflash_verify(i32(draft), D.to_device(T2, dims), tdt, B, 15, dims.vocab, acc, bon, ws(nb), nb)
    torch.cuda.synchronize()
    ps_h = ps.cpu().numpy()
    for b in sample:
        S = oracle.path_pair_scores(m, cids[b], xh[b], bids[b], 1)
        H.assert_close_rows(f"{name} pair scores b{b}", ps_h[b].reshape(-1, 16), S.reshape(-1, 16), t)
    acc_h, bon_h = acc.cpu().numpy(), bon.cpu().numpy()
    for b in range(B):
        assert (acc_h[b], bon_h[b]) == oracle.verify(draft[b], oracle.decode(T2[b], dims.dtype)), b
    say(f"  accept lengths {acc_h.tolist()[:8]}...")


def test_prefill_chunk_large_tiles():
    """A 4096-row injection at the full model shape: the context-fusion and K/V GEMMs then run
    256 x 256 tiles in their XCD-grouped order (16 x 16 and 16 x 40 tiles).  One sampled row of
    every 256-row tile (and the last row), all K/V columns of every layer, against the oracle."""
    wl, (W, m, dr) = drafter_for("c2", "config")
    dims = wl.dims
    rows, cap = 4096, wl.cap
    assert cap >= rows
    say(f"prefill chunk: {rows} rows at d {dims.d}, d_cat {dims.d_cat}")
    cache = D.KVCache(dims, 1, cap, fill=0.0)
    hid = synth.make_hidden(dims, rows, 900)
    nb = D.dflash_inject_workspace_bytes(dr.cfg, rows)
    D.dflash_inject_context(dr.cfg, dr.w, cache.kv, D.to_device(hid, dims), rows, i32([0, rows]), i32([0]),
                            i32([rows]), 1, ws(nb), nb)
    torch.cuda.synchronize()
    sample = np.array([t * 256 + (37 * t) % 256 for t in range(rows // 256)] + [rows - 1])
    _, Ko, Vo = oracle.inject_rows(m, hid[sample], sample)
    t = H.tol(dims)
    for l in range(dims.n_layers):
        Kg = cache.k[l][0].float().cpu().numpy()
        Vg = cache.vt[l][0].float().cpu().numpy()
        H.assert_close_rows(f"prefill K l{l}", Kg[:, sample].transpose(1, 0, 2), Ko[l], t)
        H.assert_close_rows(f"prefill V l{l}", Vg[:, :, sample].transpose(2, 0, 1), Vo[l], t)
