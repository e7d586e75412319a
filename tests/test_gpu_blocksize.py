"""Dynamic block size: a drafter built for blocks of 16 drafting smaller blocks (8, 5,
2 rows) matches the oracle's forward pass over that many rows, and the Path Selector
walks block_size - n_fixed positions."""
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


def ws_of(n):
    return torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")


CASES = [("t_small", 8), ("t_small", 5), ("t_conv", 5), ("t_hd128", 8), ("c1", 2), ("t_batch", 5)]


@pytest.mark.parametrize("name,bs", CASES)
def test_small_block_draft_parity(name, bs):
    say(f"draft {name} block {bs}")
    wl = synth.workload(name)
    dims = wl.dims
    W = synth.make_weights(dims, wl.seed, conv_scale="stress" if dims.use_conv else "config")
    K, V = synth.make_cache(dims, wl.ctx_lens, wl.cap, wl.seed)
    ids = synth.make_block_ids(dims, wl.batch, wl.seed, 1)       # rows >= bs are mask tokens
    B = wl.batch
    dr = D.Drafter(dims, W, block_size=bs)
    cache = D.KVCache(dims, B, wl.cap)
    cache.load_logical(K, V)
    ci = torch.zeros((B, 16, 16), dtype=torch.int32, device="cuda")
    cl = torch.zeros((B, 16, 16), dtype=torch.float32, device="cuda")
    fh = torch.zeros((B, 16, dims.d), dtype=torch.float32, device="cuda")
    lg = torch.zeros((B, 16, dims.vocab), dtype=torch.float32, device="cuda")
    nb = D.dflash_draft_workspace_bytes(dr.cfg, B, cache.cap)
    D.dflash_draft_block(dr.cfg, dr.w, cache.kv, i32(wl.ctx_lens), i32(ids), B, ci, cl, fh, lg, ws_of(nb), nb)
    torch.cuda.synchronize()
    ci, lg, fh = ci.cpu().numpy(), lg.cpu().numpy(), fh.cpu().numpy()
    m = oracle.Model(dims, W)
    t = H.tol(dims)
    for b in range(B):
        kc = [oracle.decode(K[l, b], dims.dtype) for l in range(dims.n_layers)]
        vc = [oracle.decode(V[l, b], dims.dtype) for l in range(dims.n_layers)]
        o = oracle.draft_block(m, kc, vc, int(wl.ctx_lens[b]), ids[b][:bs])
        H.assert_close_rows(f"logits b{b}", lg[b][:bs], o["logits"], t)
        H.assert_close_rows(f"final hidden b{b}", fh[b][:bs], o["xhat"], t)
        np.testing.assert_array_equal(ci[b][:bs], H.exact_topk_of(lg[b][:bs]))
        H.topk_with_margin(ci[b][:bs], o["logits"], lg[b][:bs])


@pytest.mark.parametrize("name,bs,n_fixed", [("t_small", 5, 1), ("t_small", 8, 0), ("t_f32", 2, 1)])
def test_small_block_path_parity(name, bs, n_fixed):
    say(f"path {name} block {bs} n_fixed={n_fixed}")
    wl = synth.workload(name)
    dims = wl.dims
    B = max(wl.batch, 3)
    W = synth.make_weights(dims, wl.seed, ps_scale="stress")
    ids, lg, xh = synth.make_candidates(dims, B, wl.seed)
    bids = synth.make_block_ids(dims, B, wl.seed, n_fixed)
    dr = D.Drafter(dims, W, block_size=bs)
    P = bs - n_fixed
    pidx = torch.full((B, P), -1, dtype=torch.int32, device="cuda")
    pids = torch.full((B, P), -1, dtype=torch.int32, device="cuda")
    ps = torch.zeros((B, P, 16, 16), dtype=torch.float32, device="cuda")
    nb = D.dflash_path_workspace_bytes(dr.cfg, B)
    D.dflash_select_path(dr.cfg, dr.w, i32(ids), torch.from_numpy(lg).cuda(), torch.from_numpy(xh).cuda(), i32(bids),
                         n_fixed, D.DFLASH_PATH_GREEDY, B, pidx, pids, ps, ws_of(nb), nb)
    # the sampled walk over the same scores
    u = np.random.default_rng(wl.seed).uniform(size=(B, P)).astype(np.float32)
    sidx = torch.full((B, P), -1, dtype=torch.int32, device="cuda")
    sids = torch.full((B, P), -1, dtype=torch.int32, device="cuda")
    sq = torch.zeros((B, P, 16), dtype=torch.float32, device="cuda")
    D.dflash_sample_path(dr.cfg, dr.w, i32(ids), torch.from_numpy(lg).cuda(), torch.from_numpy(xh).cuda(), i32(bids),
                         n_fixed, B, 1.0, torch.from_numpy(u).cuda(), sidx, sids, sq, None, ws_of(nb), nb)
    torch.cuda.synchronize()
    pidx, pids, ps, sidx, sq = (x.cpu().numpy() for x in (pidx, pids, ps, sidx, sq))
    m = oracle.Model(dims, W)
    for b in range(B):
        S = oracle.path_pair_scores(m, ids[b][:bs], xh[b][:bs], bids[b][:bs], n_fixed)
        assert S.shape == (P, 16, 16)
        H.assert_close_rows(f"pair scores b{b}", ps[b].reshape(-1, 16), S.reshape(-1, 16), H.tol(dims))
        lgb = lg[b, n_fixed:bs]
        np.testing.assert_array_equal(pidx[b], H.walk_f32(lgb, ps[b], n_fixed == 1, "greedy"))
        np.testing.assert_array_equal(pids[b], ids[b, n_fixed:bs][np.arange(P), pidx[b]])
        for p in range(P):
            assert sidx[b, p] == H.draw_f32(sq[b, p], u[b, p])
