"""Parity of the HIP path against the CPU oracle, element by element, on seeded inputs.

Every call goes through the C ABI (via the thin binding).  Discrete outputs are
compared bit-exactly where both sides decide on identical inputs (verification,
the path walk over the device's own pair scores, top-16 over the device's own
logits); against the oracle's independently computed floats a swap is accepted
only between entries the oracle itself ranks within twice the row's observed
error (near ties).  Continuous outputs use the row-wise tolerance of
``helpers.tol``.
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


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def ws_of(nbytes):
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")


class Ns:
    def __init__(self, **kw):
        self.__dict__.update(kw)


# ------------------------------------------------------------------ verification

VERIFY_CASES = [
    (1, 15, 151936, "bf16", 21),
    (3, 16, 3008, "bf16", 22),
    (2, 0, 1024, "f32", 23),
    (5, 7, 1040, "f32", 24),
    (32, 15, 151936, "bf16", 25),
    (4, 64, 64, "bf16", 26),
]


@pytest.mark.parametrize("B,P,V,dt,seed", VERIFY_CASES)
def test_verify_bit_exact(B, P, V, dt, seed):
    say(f"verify B={B} P={P} V={V} {dt}")
    dims = Ns(vocab=V, dtype=dt)
    rng = np.random.default_rng(seed)
    draft = rng.integers(0, V, size=(B, P)).astype(np.int32)
    T = synth.make_target_logits(dims, B, P, seed, planted="prefix", draft=draft)
    # plant exact ties at the maximum of some rows (either side of the argmax)
    flat = T.reshape(B * (P + 1), V)
    for r in range(0, flat.shape[0], 3):
        j = int(np.argmax(oracle.decode(flat[r], dt)))
        k = int(rng.integers(0, V))
        flat[r, k] = flat[r, j]
    Tg = D.to_device(T, dims)
    acc = torch.zeros(B, dtype=torch.int32, device="cuda")
    bon = torch.zeros(B, dtype=torch.int32, device="cuda")
    nb = D.dflash_verify_workspace_bytes(B, P, V)
    D.dflash_verify(dev_i32(draft) if P else None, Tg, D.DFLASH_BF16 if dt == "bf16" else D.DFLASH_F32, B, P, V,
                    acc, bon, ws_of(nb), nb)
    torch.cuda.synchronize()
    want = [oracle.verify(draft[b], oracle.decode(T[b], dt)) for b in range(B)]
    np.testing.assert_array_equal(acc.cpu().numpy(), [w[0] for w in want])
    np.testing.assert_array_equal(bon.cpu().numpy(), [w[1] for w in want])


# ------------------------------------------------------------------ injection

INJECT_CASES = ["c1", "t_small", "t_hd128", "t_f32", "t_batch"]


@pytest.mark.parametrize("name", INJECT_CASES)
def test_inject_parity(name):
    wl = synth.workload(name)
    dims = wl.dims
    say(f"inject {name}")
    W = synth.make_weights(dims, wl.seed)
    m = oracle.Model(dims, W)
    dr = D.Drafter(dims, W)
    B, cap = wl.batch, wl.cap
    rng = np.random.default_rng(wl.seed + 100)
    rows = rng.integers(1, 40, size=B)
    n_new = np.array([max(0, r - int(rng.integers(0, 3))) for r in rows], dtype=np.int32)
    pos0 = np.array([int(rng.integers(0, cap - r + 1)) for r in rows], dtype=np.int32)
    pos0[0] = cap - n_new[0]          # last rows of the cache
    row_off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    R = int(row_off[-1])
    hidden = synth.make_hidden(dims, R, wl.seed)
    cache = D.KVCache(dims, B, cap, fill=float("nan"))
    nb = D.dflash_inject_workspace_bytes(dr.cfg, R)
    D.dflash_inject_context(dr.cfg, dr.w, cache.kv, D.to_device(hidden, dims), R, dev_i32(row_off), dev_i32(pos0),
                            dev_i32(n_new), B, ws_of(nb), nb)
    torch.cuda.synchronize()
    t = H.tol(dims)
    for l in range(dims.n_layers):
        Kg, Vg = cache.logical(l)
        Kg = Kg.float().cpu().numpy()
        Vg = Vg.float().cpu().numpy()
        written = np.zeros((B, cap), dtype=bool)
        for b in range(B):
            n = int(n_new[b])
            if n == 0:
                continue
            pos = pos0[b] + np.arange(n)
            written[b, pos] = True
            _, Ko, Vo = oracle.inject_rows(m, hidden[row_off[b]:row_off[b] + n], pos)
            H.assert_close_rows(f"K l{l} b{b}", Kg[b][:, pos].transpose(1, 0, 2), Ko[l], t)
            H.assert_close_rows(f"V l{l} b{b}", Vg[b][:, pos].transpose(1, 0, 2), Vo[l], t)
        # rows outside the injected positions are untouched
        assert np.isnan(Kg[~np.broadcast_to(written[:, None, :], (B, dims.n_kv_heads, cap))]).all()
        assert np.isnan(Vg[~np.broadcast_to(written[:, None, :], (B, dims.n_kv_heads, cap))]).all()


@pytest.mark.parametrize("rows", [1, 16, 17, 32, 33, 48, 64, 65, 200])
def test_inject_row_counts(rows):
    """Every GEMM shape class: 1, 2 or 4 row tiles of the weight-streaming kernel, and the
    LDS-tiled kernel above 64 rows (with and without split-K)."""
    say(f"inject rows={rows}")
    wl = synth.workload("t_small")
    dims = wl.dims
    W = synth.make_weights(dims, wl.seed)
    m = oracle.Model(dims, W)
    dr = D.Drafter(dims, W)
    cap = ((rows + 31) // 32) * 32 + 32
    hidden = synth.make_hidden(dims, rows, wl.seed + rows)
    cache = D.KVCache(dims, 1, cap, fill=float("nan"))
    nb = D.dflash_inject_workspace_bytes(dr.cfg, rows)
    D.dflash_inject_context(dr.cfg, dr.w, cache.kv, D.to_device(hidden, dims), rows, dev_i32([0, rows]),
                            dev_i32([5]), dev_i32([rows]), 1, ws_of(nb), nb)
    torch.cuda.synchronize()
    pos = 5 + np.arange(rows)
    _, Ko, Vo = oracle.inject_rows(m, hidden, pos)
    for l in range(dims.n_layers):
        Kg, Vg = cache.logical(l)
        H.assert_close_rows(f"K l{l}", Kg.float().cpu().numpy()[0][:, pos].transpose(1, 0, 2), Ko[l], H.tol(dims))
        H.assert_close_rows(f"V l{l}", Vg.float().cpu().numpy()[0][:, pos].transpose(1, 0, 2), Vo[l], H.tol(dims))


_C2 = {}


@pytest.mark.parametrize("rows", [80, 100, 200, 256])
def test_inject_row_counts_full_width(rows):
    """The injection at the full model width (d 4096, five 4096-wide target layers): 80 and 100
    rows take one 128-row tile, 256 rows one 256-row tile, and both GEMMs split K, so their
    reductions run over one row tile of 128-column tiles (100 rows: a ragged last row group);
    200 rows take two 128-row tiles."""
    say(f"inject full width rows={rows}")
    if not _C2:
        wl = synth.workload("c2")
        _C2["wl"] = wl
        _C2["W"] = synth.make_weights(wl.dims, wl.seed)
    wl, W = _C2["wl"], _C2["W"]
    dims = wl.dims
    m = oracle.Model(dims, W)
    dr = D.Drafter(dims, W)
    cap = ((rows + 31) // 32) * 32 + 32
    hidden = synth.make_hidden(dims, rows, wl.seed + rows)
    cache = D.KVCache(dims, 1, cap, fill=float("nan"))
    nb = D.dflash_inject_workspace_bytes(dr.cfg, rows)
    D.dflash_inject_context(dr.cfg, dr.w, cache.kv, D.to_device(hidden, dims), rows, dev_i32([0, rows]),
                            dev_i32([7]), dev_i32([rows]), 1, ws_of(nb), nb)
    torch.cuda.synchronize()
    pos = 7 + np.arange(rows)
    _, Ko, Vo = oracle.inject_rows(m, hidden, pos)
    for l in range(dims.n_layers):
        Kg, Vg = cache.logical(l)
        Kg = Kg.float().cpu().numpy()[0]
        Vg = Vg.float().cpu().numpy()[0]
        H.assert_close_rows(f"K l{l}", Kg[:, pos].transpose(1, 0, 2), Ko[l], H.tol(dims))
        H.assert_close_rows(f"V l{l}", Vg[:, pos].transpose(1, 0, 2), Vo[l], H.tol(dims))
        # rows outside the written range keep the NaN fill
        keep = np.ones(cap, dtype=bool)
        keep[pos] = False
        assert np.isnan(Kg[:, keep]).all() and np.isnan(Vg[:, keep]).all(), f"layer {l}: a row outside was written"


# ------------------------------------------------------------------ drafter forward

DRAFT_CASES = ["c1", "t_small", "t_conv", "t_hd128", "t_f32", "t_batch"]


def run_draft(dims, dr, cache, ctx_lens, ids):
    B = len(ctx_lens)
    M = 16 * B
    ci = torch.zeros((B, 16, 16), dtype=torch.int32, device="cuda")
    cl = torch.zeros((B, 16, 16), dtype=torch.float32, device="cuda")
    fh = torch.zeros((B, 16, dims.d), dtype=torch.float32, device="cuda")
    lg = torch.zeros((B, 16, dims.vocab), dtype=torch.float32, device="cuda")
    nb = D.dflash_draft_workspace_bytes(dr.cfg, B, cache.cap)
    D.dflash_draft_block(dr.cfg, dr.w, cache.kv, dev_i32(ctx_lens), dev_i32(ids), B, ci, cl, fh, lg, ws_of(nb), nb)
    torch.cuda.synchronize()
    return ci.cpu().numpy(), cl.cpu().numpy(), fh.cpu().numpy(), lg.cpu().numpy()


def draft_setup(name, poison=False, n_fixed=1):
    wl = synth.workload(name)
    dims = wl.dims
    W = synth.make_weights(dims, wl.seed, conv_scale="stress" if dims.use_conv else "config")
    K, V = synth.make_cache(dims, wl.ctx_lens, wl.cap, wl.seed, poison=poison)
    ids = synth.make_block_ids(dims, wl.batch, wl.seed, n_fixed)
    return wl, dims, W, K, V, ids


@pytest.mark.parametrize("name", DRAFT_CASES)
def test_draft_parity(name):
    say(f"draft {name}")
    wl, dims, W, K, V, ids = draft_setup(name)
    dr = D.Drafter(dims, W)
    cache = D.KVCache(dims, wl.batch, wl.cap)
    cache.load_logical(K, V)
    ci, cl, fh, lg = run_draft(dims, dr, cache, wl.ctx_lens, ids)
    m = oracle.Model(dims, W)
    outs = H.oracle_draft(m, K, V, wl.ctx_lens, ids)
    t = H.tol(dims)
    near = 0
    for b, o in enumerate(outs):
        H.assert_close_rows(f"logits b{b}", lg[b], o["logits"], t)
        H.assert_close_rows(f"final hidden b{b}", fh[b], o["xhat"], t)
        # top-16 is exactly the stable sort of the device's own logits
        np.testing.assert_array_equal(ci[b], H.exact_topk_of(lg[b]))
        np.testing.assert_array_equal(cl[b], np.take_along_axis(lg[b], ci[b].astype(np.int64), axis=1))
        near += H.topk_with_margin(ci[b], o["logits"], lg[b])
    say(f"  near-tie top-16 swaps: {near}")


@pytest.mark.parametrize("batch,vocab,period", [(12, 2000, 0), (12, 2000, 37), (32, 32848, 37)])
def test_draft_top16_over_group_maxima(batch, vocab, period):
    """Several drafted blocks with an unsplit LM head: the top-16 stage reads only the
    128-column groups whose maximum reaches the 16th-largest group maximum.  Vocabularies
    that end in a partial group (and, at 512 rows with 256-column tiles, a tile whose second
    half lies wholly past the vocabulary); with period > 0 the LM-head rows repeat, so every
    logit value recurs across many groups and the ties must resolve to the lowest ids."""
    import dataclasses
    say(f"draft top-16 over group maxima: batch {batch}, vocab {vocab}, period {period}")
    base = synth.workload("t_batch")
    dims = dataclasses.replace(base.dims, vocab=vocab)
    ctx = tuple((17 * i) % 150 for i in range(batch))
    cap = ((max(ctx) + 16 + 31) // 32) * 32
    W = synth.make_weights(dims, base.seed + period)
    if period:
        lm = W["lm_head"]
        W["lm_head"] = lm[np.arange(lm.shape[0]) % period].copy()
    K, V = synth.make_cache(dims, ctx, cap, base.seed + 2)
    ids = synth.make_block_ids(dims, batch, base.seed, 1)
    dr = D.Drafter(dims, W)
    cache = D.KVCache(dims, batch, cap)
    cache.load_logical(K, V)
    ci, cl, fh, lg = run_draft(dims, dr, cache, ctx, ids)
    for b in range(batch):
        np.testing.assert_array_equal(ci[b], H.exact_topk_of(lg[b]))
        np.testing.assert_array_equal(cl[b], np.take_along_axis(lg[b], ci[b].astype(np.int64), axis=1))
    if period:   # the winners of a row all carry its largest value, at the lowest ids
        assert (cl == cl[..., :1]).all()
    outs = H.oracle_draft(oracle.Model(dims, W), K, V, ctx, ids)
    for b in (0, batch - 1):
        H.assert_close_rows(f"logits b{b}", lg[b], outs[b]["logits"], H.tol(dims))


def test_draft_parity_256_rows():
    """Sixteen drafted blocks (256 rows: the pipelined GEMM's 256-row tiles on every
    projection) with the dynamic short conv and the context gate, ragged contexts including
    an empty one; every sequence against the oracle."""
    base = synth.workload("t_conv")
    dims = base.dims
    B = 16
    ctx = tuple((37 * i + 5) % 260 if i else 0 for i in range(B))
    cap = ((max(ctx) + 16 + 31) // 32) * 32
    say(f"draft 256 rows (t_conv dims): contexts {list(ctx)}")
    W = synth.make_weights(dims, base.seed + 3, conv_scale="stress")
    K, V = synth.make_cache(dims, ctx, cap, base.seed + 4)
    ids = synth.make_block_ids(dims, B, base.seed + 5, 1)
    dr = D.Drafter(dims, W)
    cache = D.KVCache(dims, B, cap)
    cache.load_logical(K, V)
    ci, cl, fh, lg = run_draft(dims, dr, cache, ctx, ids)
    outs = H.oracle_draft(oracle.Model(dims, W), K, V, ctx, ids)
    t = H.tol(dims)
    near = 0
    for b, o in enumerate(outs):
        H.assert_close_rows(f"logits b{b}", lg[b], o["logits"], t)
        H.assert_close_rows(f"final hidden b{b}", fh[b], o["xhat"], t)
        np.testing.assert_array_equal(ci[b], H.exact_topk_of(lg[b]))
        near += H.topk_with_margin(ci[b], o["logits"], lg[b])
    say(f"  near-tie top-16 swaps: {near}")


def test_draft_long_context():
    """Contexts long enough for many 32-key slabs per attention split (and ragged ends)."""
    say("draft long context t_hd128")
    wl = synth.workload("t_hd128")
    dims = wl.dims
    ctx = (9000, 4097)
    cap = ((max(ctx) + 16 + 31) // 32) * 32
    W = synth.make_weights(dims, wl.seed)
    K, V = synth.make_cache(dims, ctx, cap, wl.seed + 1)
    ids = synth.make_block_ids(dims, len(ctx), wl.seed, 1)
    dr = D.Drafter(dims, W)
    cache = D.KVCache(dims, len(ctx), cap)
    cache.load_logical(K, V)
    ci, cl, fh, lg = run_draft(dims, dr, cache, ctx, ids)
    outs = H.oracle_draft(oracle.Model(dims, W), K, V, ctx, ids)
    for b, o in enumerate(outs):
        H.assert_close_rows(f"logits b{b}", lg[b], o["logits"], H.tol(dims))
        H.assert_close_rows(f"final hidden b{b}", fh[b], o["xhat"], H.tol(dims))


def test_draft_ignores_rows_beyond_context():
    say("draft poison t_small")
    wl, dims, W, K, V, ids = draft_setup("t_small")
    _, _, _, Kp, Vp, _ = draft_setup("t_small", poison=True)
    dr = D.Drafter(dims, W)
    a = D.KVCache(dims, wl.batch, wl.cap)
    a.load_logical(K, V)
    p = D.KVCache(dims, wl.batch, wl.cap)
    p.load_logical(Kp, Vp)
    ra = run_draft(dims, dr, a, wl.ctx_lens, ids)
    rp = run_draft(dims, dr, p, wl.ctx_lens, ids)
    for x, y in zip(ra, rp):
        assert np.isfinite(y.astype(np.float64)).all()
        np.testing.assert_array_equal(x, y)


def test_draft_deterministic():
    say("draft determinism t_conv")
    wl, dims, W, K, V, ids = draft_setup("t_conv")
    dr = D.Drafter(dims, W)
    c = D.KVCache(dims, wl.batch, wl.cap)
    c.load_logical(K, V)
    r1 = run_draft(dims, dr, c, wl.ctx_lens, ids)
    r2 = run_draft(dims, dr, c, wl.ctx_lens, ids)
    for x, y in zip(r1, r2):
        np.testing.assert_array_equal(x, y)


# ------------------------------------------------------------------ Path Selector

PATH_CASES = [("t_small", 1, "greedy"), ("t_small", 0, "greedy"), ("t_conv", 1, "greedy"), ("t_conv", 1, "exact"),
              ("t_hd128", 0, "exact"), ("t_f32", 1, "greedy"), ("t_f32", 0, "exact"), ("c1", 1, "greedy")]


@pytest.mark.parametrize("name,n_fixed,mode", PATH_CASES)
def test_path_parity(name, n_fixed, mode):
    say(f"path {name} n_fixed={n_fixed} {mode}")
    wl = synth.workload(name)
    dims = wl.dims
    B = max(wl.batch, 3)
    W = synth.make_weights(dims, wl.seed, ps_scale="stress")
    ids, lg, xh = synth.make_candidates(dims, B, wl.seed)
    bids = synth.make_block_ids(dims, B, wl.seed, n_fixed)
    dr = D.Drafter(dims, W)
    P = 16 - n_fixed
    pidx = torch.zeros((B, P), dtype=torch.int32, device="cuda")
    pids = torch.zeros((B, P), dtype=torch.int32, device="cuda")
    ps = torch.zeros((B, P, 16, 16), dtype=torch.float32, device="cuda")
    nb = D.dflash_path_workspace_bytes(dr.cfg, B)
    D.dflash_select_path(dr.cfg, dr.w, dev_i32(ids), torch.from_numpy(lg).cuda(), torch.from_numpy(xh).cuda(),
                         dev_i32(bids), n_fixed, D.DFLASH_PATH_GREEDY if mode == "greedy" else D.DFLASH_PATH_EXACT,
                         B, pidx, pids, ps, ws_of(nb), nb)
    torch.cuda.synchronize()
    pidx, pids, ps = pidx.cpu().numpy(), pids.cpu().numpy(), ps.cpu().numpy()
    m = oracle.Model(dims, W)
    t = H.tol(dims)
    moved = 0
    for b in range(B):
        S = oracle.path_pair_scores(m, ids[b], xh[b], bids[b], n_fixed)
        H.assert_close_rows(f"pair scores b{b}", ps[b].reshape(-1, 16), S.reshape(-1, 16), t)
        lgb = lg[b, n_fixed:]
        # the device path is exactly the walk over its own scores
        np.testing.assert_array_equal(pidx[b], H.walk_f32(lgb, ps[b], n_fixed == 1, mode))
        np.testing.assert_array_equal(pids[b], ids[b, n_fixed:][np.arange(P), pidx[b]])
        # against the oracle's own scores: equal, or a near tie
        oidx, otot = oracle.select_path(lgb, S, n_fixed == 1, mode)
        if not np.array_equal(oidx, pidx[b]):
            margin = 2 * P * np.abs(ps[b] - S).max() + 1e-6
            gtot = lgb[0, pidx[b][0]] + (S[0, 0, pidx[b][0]] if n_fixed else 0) + sum(
                lgb[p, pidx[b][p]] + S[p, pidx[b][p - 1], pidx[b][p]] for p in range(1, P))
            if mode == "exact":
                assert otot - gtot <= margin, (otot, gtot, margin)
            else:
                p0 = int(np.flatnonzero(oidx != pidx[b])[0])
                prev = pidx[b][p0 - 1] if p0 > 0 else 0
                sc = lgb[p0] + (S[p0, prev] if (p0 > 0 or n_fixed) else 0)
                assert sc[oidx[p0]] - sc[pidx[b][p0]] <= margin
            moved += 1
    say(f"  near-tie path differences: {moved}")


@pytest.mark.parametrize("name", ["t_small", "t_conv"])
def test_path_table_and_projection_agree(name):
    """The per-token table (built once) and the projection of the candidates' embeddings
    at each call give the same pair scores (fp32 sums in different orders) and paths."""
    say(f"path table vs projection {name}")
    wl = synth.workload(name)
    dims = wl.dims
    B = 4
    W = synth.make_weights(dims, wl.seed, ps_scale="stress")
    ids, lg, xh = synth.make_candidates(dims, B, wl.seed + 5)
    bids = synth.make_block_ids(dims, B, wl.seed + 5, 1)
    outs = []
    for table in (True, False):
        dr = D.Drafter(dims, W, path_table=table)
        assert (dr.table is not None) == table
        pidx = torch.zeros((B, 15), dtype=torch.int32, device="cuda")
        pids = torch.zeros((B, 15), dtype=torch.int32, device="cuda")
        ps = torch.zeros((B, 15, 16, 16), dtype=torch.float32, device="cuda")
        nb = D.dflash_path_workspace_bytes(dr.cfg, B)
        D.dflash_select_path(dr.cfg, dr.w, dev_i32(ids), torch.from_numpy(lg).cuda(), torch.from_numpy(xh).cuda(),
                             dev_i32(bids), 1, D.DFLASH_PATH_GREEDY, B, pidx, pids, ps, ws_of(nb), nb)
        torch.cuda.synchronize()
        outs.append((pidx.cpu().numpy(), ps.cpu().numpy()))
    assert H.rowwise_relerr(outs[0][1].reshape(-1, 16), outs[1][1].reshape(-1, 16)) < 1e-5
    for b in range(B):
        np.testing.assert_array_equal(outs[0][0][b], H.walk_f32(lg[b, 1:], outs[0][1][b], True, "greedy"))
        np.testing.assert_array_equal(outs[1][0][b], H.walk_f32(lg[b, 1:], outs[1][1][b], True, "greedy"))


# ------------------------------------------------------------------ whole step (tiny workload)

@pytest.mark.parametrize("name", ["c1", "t_conv"])
def test_step_end_to_end(name):
    say(f"step {name}")
    wl = synth.workload(name)
    dims = wl.dims
    W = synth.make_weights(dims, wl.seed, ps_scale="stress")
    B, cap = wl.batch, wl.cap
    ctx = np.asarray(wl.ctx_lens, dtype=np.int32)
    # prefill: inject every context row from target hiddens
    row_off, pos0, n_new = synth.make_prefill_positions(ctx)
    R = int(row_off[-1])
    hidden = synth.make_hidden(dims, max(R, 1), wl.seed, key=1)
    dr = D.Drafter(dims, W)
    cache = D.KVCache(dims, B, cap)
    if R:
        nb = D.dflash_inject_workspace_bytes(dr.cfg, R)
        D.dflash_inject_context(dr.cfg, dr.w, cache.kv, D.to_device(hidden, dims), R, dev_i32(row_off),
                                dev_i32(pos0), dev_i32(n_new), B, ws_of(nb), nb)
    ids = synth.make_block_ids(dims, B, wl.seed, 1)
    ci, cl, fh, lg = run_draft(dims, dr, cache, ctx, ids)
    P = 15
    pidx = torch.zeros((B, P), dtype=torch.int32, device="cuda")
    pids = torch.zeros((B, P), dtype=torch.int32, device="cuda")
    nb = D.dflash_path_workspace_bytes(dr.cfg, B)
    D.dflash_select_path(dr.cfg, dr.w, dev_i32(ci), torch.from_numpy(cl).cuda(), torch.from_numpy(fh).cuda(),
                         dev_i32(ids), 1, D.DFLASH_PATH_GREEDY, B, pidx, pids, None, ws_of(nb), nb)
    T = synth.make_target_logits(dims, B, P, wl.seed, planted="random")
    acc = torch.zeros(B, dtype=torch.int32, device="cuda")
    bon = torch.zeros(B, dtype=torch.int32, device="cuda")
    nb = D.dflash_verify_workspace_bytes(B, P, dims.vocab)
    D.dflash_verify(pids, D.to_device(T, dims), D.DFLASH_BF16 if dims.dtype == "bf16" else D.DFLASH_F32, B, P,
                    dims.vocab, acc, bon, ws_of(nb), nb)
    torch.cuda.synchronize()
    m = oracle.Model(dims, W)
    t = H.tol(dims)
    for b in range(B):
        L = int(ctx[b])
        kc = [np.zeros((dims.n_kv_heads, cap, dims.head_dim)) for _ in range(dims.n_layers)]
        vc = [np.zeros((dims.n_kv_heads, cap, dims.head_dim)) for _ in range(dims.n_layers)]
        o = oracle.drafting_step(m, kc, vc, L, hidden[row_off[b]:row_off[b + 1]], np.arange(L), ids[b],
                                 oracle.decode(T[b], dims.dtype))
        H.assert_close_rows(f"logits b{b}", lg[b], o["logits"], t)
        H.topk_with_margin(ci[b], o["logits"], lg[b])
        gp = pids.cpu().numpy()[b]
        # the device's verification of its own path is valid for the same target logits
        Tf = oracle.decode(T[b], dims.dtype)
        assert (int(acc[b]), int(bon[b])) == H.accept_of(gp, Tf)
        # where both sides reach the same candidates and path, the outcomes agree
        if np.array_equal(ci[b], o["cand_ids"]) and np.array_equal(gp, o["path_ids"]):
            assert (int(acc[b]), int(bon[b])) == (o["accept_len"], o["bonus"])
