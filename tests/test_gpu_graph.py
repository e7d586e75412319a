"""The drafting step captured in a HIP graph.

A serving loop captures inject -> draft -> path -> verify once and replays it.  The four
calls allocate nothing, synchronise nothing and record no memory fills, so the captured
step must equal the eager one bit for bit on every replay (each replay re-injects the same
verified rows, so the cache state does not drift; the target logits favour a seeded prefix of
the drafted path, so the accepted lengths vary).  Replays are interleaved with eager work
and synchronisations, and every output is cleared between them."""
import sys

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
import block_diffusion_drafter_feature_amd as D  # noqa: E402


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def ws_of(nbytes):
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("name", ["t_conv", "t_small", "c1", "c2"])
def test_step_graph_replays(name):
    wl = synth.workload(name)
    dims = wl.dims
    B, cap = wl.batch, wl.cap
    say(f"graph step {name}: batch {B}, contexts {list(wl.ctx_lens)}")
    W = synth.make_weights(dims, wl.seed, ps_scale="stress")
    ctx = np.asarray(wl.ctx_lens, dtype=np.int32)
    dr = D.Drafter(dims, W)
    cache = D.KVCache(dims, B, cap)
    # prefill (eager): every context row
    row_off, pos0, n_new = synth.make_prefill_positions(ctx)
    R = int(row_off[-1])
    if R:
        hid = synth.make_hidden(dims, R, wl.seed, key=1)
        nb = D.dflash_inject_workspace_bytes(dr.cfg, R)
        D.dflash_inject_context(dr.cfg, dr.w, cache.kv, D.to_device(hid, dims), R, dev_i32(row_off),
                                dev_i32(pos0), dev_i32(n_new), B, ws_of(nb), nb)
    # the step's inputs: the last (up to) 16 verified rows of each sequence again
    s_new = np.minimum(ctx, 16).astype(np.int32)
    s_pos0 = (ctx - s_new).astype(np.int32)
    s_off = np.zeros(B + 1, dtype=np.int32)
    s_off[1:] = np.cumsum(s_new)
    RS = max(int(s_off[-1]), 1)
    hidden = D.to_device(synth.make_hidden(dims, RS, wl.seed + 7, key=2), dims)
    off_t, pos_t, new_t, ctx_t = dev_i32(s_off), dev_i32(s_pos0), dev_i32(s_new), dev_i32(ctx)
    ids_t = dev_i32(synth.make_block_ids(dims, B, wl.seed, 1))
    P = 15
    T = D.to_device(synth.make_target_logits(dims, B, P, wl.seed, planted="random"), dims)
    tdt = D.DFLASH_BF16 if dims.dtype == "bf16" else D.DFLASH_F32
    out = dict(ci=torch.zeros((B, 16, 16), dtype=torch.int32, device="cuda"),
               cl=torch.zeros((B, 16, 16), dtype=torch.float32, device="cuda"),
               fh=torch.zeros((B, 16, dims.d), dtype=torch.float32, device="cuda"),
               lg=torch.zeros((B, 16, dims.vocab), dtype=torch.float32, device="cuda"),
               pidx=torch.zeros((B, P), dtype=torch.int32, device="cuda"),
               pids=torch.zeros((B, P), dtype=torch.int32, device="cuda"),
               acc=torch.zeros(B, dtype=torch.int32, device="cuda"),
               bon=torch.zeros(B, dtype=torch.int32, device="cuda"))
    nbi = D.dflash_inject_workspace_bytes(dr.cfg, RS)
    nbd = D.dflash_draft_workspace_bytes(dr.cfg, B, cap)
    nbp = D.dflash_path_workspace_bytes(dr.cfg, B)
    nbv = D.dflash_verify_workspace_bytes(B, P, dims.vocab)
    wsi, wsd, wsp, wsv = ws_of(nbi), ws_of(nbd), ws_of(nbp), ws_of(nbv)

    def step():
        D.dflash_inject_context(dr.cfg, dr.w, cache.kv, hidden, RS, off_t, pos_t, new_t, B, wsi, nbi)
        D.dflash_draft_block(dr.cfg, dr.w, cache.kv, ctx_t, ids_t, B, out["ci"], out["cl"], out["fh"], out["lg"],
                             wsd, nbd)
        D.dflash_select_path(dr.cfg, dr.w, out["ci"], out["cl"], out["fh"], ids_t, 1, D.DFLASH_PATH_GREEDY, B,
                             out["pidx"], out["pids"], None, wsp, nbp)
        D.dflash_verify(out["pids"], T, tdt, B, P, dims.vocab, out["acc"], out["bon"], wsv, nbv)

    def snapshot():
        torch.cuda.synchronize()
        snap = {k: v.clone() for k, v in out.items()}
        for l in range(dims.n_layers):
            snap[f"k{l}"] = cache.k[l].clone()
            snap[f"vt{l}"] = cache.vt[l].clone()
        return snap

    step()
    # the target then favours a seeded prefix of the drafted path, so verification accepts a
    # seeded number of drafts (the same in every replay: the path does not change)
    torch.cuda.synchronize()
    Tp = synth.make_target_logits(dims, B, P, wl.seed, planted="prefix", draft=out["pids"].cpu().numpy(), boost=8.0)
    T.copy_(D.to_device(Tp, dims))
    step()
    ref = snapshot()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()   # warm-up on the capturing stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    junk = torch.randn(512, 512, device="cuda")
    for r in range(3):
        for v in out.values():
            v.zero_()
        junk = junk @ junk.t()          # eager work between replays
        junk /= junk.norm()
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for k, v in ref.items():
            assert torch.equal(got[k], v), f"replay {r}: {k} differs from the eager step"
    say(f"  3 replays equal the eager step (accepted {ref['acc'].tolist()})")
