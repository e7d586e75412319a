"""FP8 weight storage on the device: the quantizer bit-exact against the oracle's, and
the drafting step with E4M3 projections against the oracle's model of the same
quantized weights (both GEMM paths: weight streaming for one block, the pipelined
kernel for batches)."""
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


@pytest.mark.parametrize("rows,cols", [(300, 256), (16, 4096), (5, 64)])
def test_quantize_bit_exact(rows, cols):
    say(f"quantize {rows}x{cols}")
    r = np.random.default_rng(rows + cols)
    w = (r.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    w[0] = 0.0                                     # zero row
    if rows > 2:
        w[1] = 0.0
        w[1, 7] = 3.0                              # one nonzero element
    if rows > 3:
        # power-of-two scale (amax = 448 * 2^-10): w / scale is exact, so grid midpoints
        # (ties) and values below 2^-6 (subnormal codes) are hit exactly
        grid = oracle.e4m3_values()[:127]
        mids = (grid[:-1] + grid[1:]) / 2
        vals = np.concatenate([grid, mids, -mids])[:cols] * 2.0 ** -10
        w[2, :] = 0.0
        w[2, :len(vals)] = vals
        w[2, -1] = 448.0 * 2.0 ** -10
    bits = synth.f32_to_bf16_bits(w)
    wf = synth.bits_to_f32(bits)
    codes, scale = oracle.quantize_fp8_rows(wf)
    out = torch.full((rows * (cols + 16),), 0xAB, dtype=torch.uint8, device="cuda")
    D.dflash_quantize_fp8(D.to_device(bits, synth.workload("t_small").dims), rows, cols, out)
    torch.cuda.synchronize()
    o = out.cpu().numpy().reshape(rows, cols + 16)
    np.testing.assert_array_equal(o[:, :cols], codes)
    np.testing.assert_array_equal(o[:, cols:cols + 4].copy().view(np.float32)[:, 0], scale)
    assert (o[:, cols + 4:] == 0).all()


def fp8_setup(name, batch=None):
    wl = synth.workload(name)
    dims = wl.dims
    ctx = tuple(wl.ctx_lens[:batch] if batch else wl.ctx_lens)
    B = len(ctx)
    W = synth.make_weights(dims, wl.seed, conv_scale="stress" if dims.use_conv else "config")
    K, V = synth.make_cache(dims, ctx, wl.cap, wl.seed)
    ids = synth.make_block_ids(dims, B, wl.seed, 1)
    return wl, dims, W, K, V, ids, ctx


FP8_DRAFT = [("t_small", None), ("t_small", 1), ("t_conv", None), ("t_hd128", 1), ("t_batch", None)]


@pytest.mark.parametrize("name,batch", FP8_DRAFT)
def test_fp8_draft_parity(name, batch):
    wl, dims, W, K, V, ids, ctx = fp8_setup(name, batch)
    B = len(ctx)
    say(f"fp8 draft {name} batch {B}")
    dr = D.Drafter(dims, W, fp8=True)
    cache = D.KVCache(dims, B, wl.cap)
    cache.load_logical(K, V)
    ci = torch.zeros((B, 16, 16), dtype=torch.int32, device="cuda")
    cl = torch.zeros((B, 16, 16), dtype=torch.float32, device="cuda")
    fh = torch.zeros((B, 16, dims.d), dtype=torch.float32, device="cuda")
    lg = torch.zeros((B, 16, dims.vocab), dtype=torch.float32, device="cuda")
    nb = D.dflash_draft_workspace_bytes(dr.cfg, B, cache.cap)
    D.dflash_draft_block(dr.cfg, dr.w, cache.kv, i32(ctx), i32(ids), B, ci, cl, fh, lg, ws_of(nb), nb)
    torch.cuda.synchronize()
    ci, lg, fh = ci.cpu().numpy(), lg.cpu().numpy(), fh.cpu().numpy()
    m8 = oracle.Model(dims, W, fp8=True)
    outs = H.oracle_draft(m8, K, V, ctx, ids)
    t = H.tol(dims)
    m16 = oracle.Model(dims, W)
    for b, o in enumerate(outs):
        e = H.assert_close_rows(f"logits b{b}", lg[b], o["logits"], t)
        H.assert_close_rows(f"final hidden b{b}", fh[b], o["xhat"], t)
        np.testing.assert_array_equal(ci[b], H.exact_topk_of(lg[b]))
        # the quantization is visible: the bf16-weight oracle is measurably further away
        o16 = oracle.draft_block(m16, [oracle.decode(K[l, b], dims.dtype) for l in range(dims.n_layers)],
                                 [oracle.decode(V[l, b], dims.dtype) for l in range(dims.n_layers)], int(ctx[b]),
                                 ids[b])
        e16 = H.rowwise_relerr(lg[b], o16["logits"])
        say(f"  b{b}: logits rel err {e:.2e} against the fp8 oracle, {e16:.2e} against the bf16 one")
        assert e16 > e


def test_fp8_draft_wide_vocab_256_rows():
    """Sixteen drafted blocks (256 rows, the pipelined kernel's 256-row tiles) over a
    vocabulary of 65552 columns, the last tile holding 16 live columns: logits against the
    oracle's quantized model, top-16 exactly that of the device's logits."""
    import dataclasses
    base = synth.workload("t_batch")
    dims = dataclasses.replace(base.dims, vocab=65552)
    B = 16
    ctx = tuple((23 * i) % 190 for i in range(B))
    cap = ((max(ctx) + 16 + 31) // 32) * 32
    say(f"fp8 draft wide vocab: batch {B}, vocab {dims.vocab}")
    W = synth.make_weights(dims, base.seed + 5)
    K, V = synth.make_cache(dims, ctx, cap, base.seed + 6)
    ids = synth.make_block_ids(dims, B, base.seed, 1)
    dr = D.Drafter(dims, W, fp8=True)
    cache = D.KVCache(dims, B, cap)
    cache.load_logical(K, V)
    ci = torch.zeros((B, 16, 16), dtype=torch.int32, device="cuda")
    cl = torch.zeros((B, 16, 16), dtype=torch.float32, device="cuda")
    fh = torch.zeros((B, 16, dims.d), dtype=torch.float32, device="cuda")
    lg = torch.zeros((B, 16, dims.vocab), dtype=torch.float32, device="cuda")
    nb = D.dflash_draft_workspace_bytes(dr.cfg, B, cache.cap)
    D.dflash_draft_block(dr.cfg, dr.w, cache.kv, i32(ctx), i32(ids), B, ci, cl, fh, lg, ws_of(nb), nb)
    torch.cuda.synchronize()
    ci, cl, lg = ci.cpu().numpy(), cl.cpu().numpy(), lg.cpu().numpy()
    for b in range(B):
        np.testing.assert_array_equal(ci[b], H.exact_topk_of(lg[b]))
        np.testing.assert_array_equal(cl[b], np.take_along_axis(lg[b], ci[b].astype(np.int64), axis=1))
    sel = (0, 7, B - 1)
    outs = H.oracle_draft(oracle.Model(dims, W, fp8=True), K[:, list(sel)], V[:, list(sel)],
                          tuple(ctx[b] for b in sel), ids[list(sel)])
    for b, o in zip(sel, outs):
        e = H.assert_close_rows(f"logits b{b}", lg[b], o["logits"], H.tol(dims))
        say(f"  b{b}: logits rel err {e:.2e}")


@pytest.mark.parametrize("rows", [16, 200])
def test_fp8_inject_parity(rows):
    say(f"fp8 inject rows={rows}")
    wl = synth.workload("t_small")
    dims = wl.dims
    W = synth.make_weights(dims, wl.seed)
    m = oracle.Model(dims, W, fp8=True)
    dr = D.Drafter(dims, W, fp8=True)
    cap = ((rows + 31) // 32) * 32 + 32
    hidden = synth.make_hidden(dims, rows, wl.seed + rows)
    cache = D.KVCache(dims, 1, cap, fill=float("nan"))
    nb = D.dflash_inject_workspace_bytes(dr.cfg, rows)
    D.dflash_inject_context(dr.cfg, dr.w, cache.kv, D.to_device(hidden, dims), rows, i32([0, rows]), i32([5]),
                            i32([rows]), 1, ws_of(nb), nb)
    torch.cuda.synchronize()
    pos = 5 + np.arange(rows)
    _, Ko, Vo = oracle.inject_rows(m, hidden, pos)
    for l in range(dims.n_layers):
        Kg, Vg = cache.logical(l)
        H.assert_close_rows(f"K l{l}", Kg.float().cpu().numpy()[0][:, pos].transpose(1, 0, 2), Ko[l], H.tol(dims))
        H.assert_close_rows(f"V l{l}", Vg.float().cpu().numpy()[0][:, pos].transpose(1, 0, 2), Vo[l], H.tol(dims))
