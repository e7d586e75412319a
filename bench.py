#!/usr/bin/env python3
"""Throughput of one DFlash-style drafting step on one MI355X: drafted 16-token blocks/s.

A step is one pass of the whole hot path over one batch of synthetic inputs already
resident in HBM:
  1. dflash_inject_context : inject 16 new context rows per sequence (positions L-16..L-1)
  2. dflash_draft_block    : one parallel forward pass over the 16-row block
  3. dflash_select_path    : Path Selector pair scores + greedy path
  4. dflash_verify         : greedy acceptance against the target logits
blocks/s = batch x steps/s.  The default workload is the full DFlash 2 step (``--workload
c5``: batch 16, context 16384, the Qwen3-8B-shaped drafter with the dynamic short conv around
every sublayer and the gated Path Selector), the largest configuration that runs on one GPU
and the only one with every part of the step; c1..c4 select the other shapes.  Before the
timed steps the whole context of every sequence is injected (prefill), and that injection is
timed on its own (rows/s and the matrix-core fraction of its GEMMs).

Prints ONE JSON line (rank 0): the metric, a roofline object for the dominant kernel
(algorithmic bytes or flops per launch over its event-timed duration inside the timed
region), the per-kernel breakdown, and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12            # MI355X HBM3E, bytes/s
MFMA_PEAK = {"bf16": 2.5e15, "f32": 157.3e12}   # dense matrix-core peaks (fp32: vector/matrix fp32)
METRIC = "drafted 16-token blocks/sec at 1 GPU; attention HBM GB/s and GEMM MFMA % of peak"


PROBE_EVERY = 10   # timed steps per probed step


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c5", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU oracle sample budget (0 to skip)")
    ap.add_argument("--no-breakdown", action="store_true", help="skip the per-kernel breakdown pass")
    ap.add_argument("--cycles", type=int, default=32,
                    help="also time this many full drafting cycles (inject the accepted rows with counts read "
                         "on the device, draft, path, verify, advance) and report tau and tokens/s")
    ap.add_argument("--sampled-steps", type=int, default=20,
                    help="also time this many steps of the sampling variant (sampled path choice and "
                         "verification by rejection sampling, temperature 0.8) and report them apart")
    ap.add_argument("--graph-steps", type=int, default=20,
                    help="also capture the step in a HIP graph and time this many replays (reported apart)")
    ap.add_argument("--fp8-steps", type=int, default=20,
                    help="also time this many steps with the streamed projections in FP8 storage (E4M3 codes, "
                         "a float32 scale per row) and report them apart (bf16 workloads)")
    ap.add_argument("--block-sizes", default="8,5",
                    help="also time the step with these smaller drafted blocks (dynamic block size; comma list, "
                         "empty to skip)")
    ap.add_argument("--cal-dim", type=int, default=256,
                    help="also time the bonus-guided calibration (MLP of this hidden width, device-drawn "
                         "N(0, 0.02^2) weights) on the step's drafted block; 0 to skip")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the step, run a plain fp32 elementwise copy (torch.neg) of this many MiB "
                         "three times: a kernel of known traffic that calibrates HBM byte counters")
    ap.add_argument("--prefill", choices=["inject", "synthetic"], default="inject",
                    help="fill the KV cache by injecting every context row (default; timed apart) or with "
                         "device-generated values at the scale injection produces")
    return ap.parse_args()


# ------------------------------------------------------------------ algorithmic work per probed kernel

def kernel_work(dims, batch, ctx_lens, fp8=False, lists=0):
    """(bytes, flops) each probed kernel must move / compute at minimum, per launch.  With
    fp8, the streamed projections are read in FP8 storage (cols + 16 bytes per row).  With
    lists > 0 the LM head keeps per-work-group top-16 lists instead of writing the logits
    (one drafted block, bf16 weights): it writes lists x 16 (value, id) pairs per row, which
    the top-16 merge reads back."""
    e = 2 if dims.dtype == "bf16" else 4
    d, H, Hkv, hd, F, V = dims.d, dims.n_heads, dims.n_kv_heads, dims.head_dim, dims.d_ffn, dims.vocab
    M = 16 * batch
    hq, hk = H * hd, Hkv * hd
    kv_rows = sum(ctx_lens)

    def wb(rows, cols):
        return rows * (cols + 16) if fp8 else rows * cols * e
    w = {
        "lm_head": (wb(V, d) + M * d * e + (M * lists * 16 * 8 if lists else M * V * 4), 2 * M * V * d),
        "qkv": (wb(hq + 2 * hk, d) + M * d * e + M * (hq + 2 * hk) * e, 2 * M * (hq + 2 * hk) * d),
        "o": (wb(d, hq) + M * hq * e + 2 * M * d * 4, 2 * M * d * hq),
        "gate_up": (wb(2 * F, d) + M * d * e + M * F * e, 2 * M * 2 * F * d),
        "down": (wb(d, F) + M * F * e + 2 * M * d * 4, 2 * M * d * F),
        # block attention of one layer: every context K and V row once, plus q, block k/v, o
        "attn": (2 * kv_rows * hk * e + M * hq * e * 2 + 2 * M * hk * e,
                 2 * 2 * batch * 16 * H * hd * (sum(ctx_lens) / max(batch, 1) + 16)),
        "topk": (M * lists * 16 * 8 if lists else M * V * 4, 0),
        "inject_fc": (wb(d, dims.d_cat) + M * dims.d_cat * e + M * d * 4, 2 * M * d * dims.d_cat),
        "inject_kv": (dims.n_layers * wb(2 * hk, d) + M * d * e + M * dims.n_layers * 2 * hk * e,
                      2 * M * dims.n_layers * 2 * hk * d),
    }
    if dims.use_conv:
        ng = d // 16
        gen = 2 * ng * d * e + 2 * d * e              # correction generator + two static taps
        # FFN input site: the residual rows in, the norm gain, the conv'd rows out (GEMM operand)
        w["conv_pre"] = (gen + M * d * 4 + d * e + M * d * e, 2 * M * 2 * ng * d)
        # attention output site: the O projection's rows in, the residual read and written
        w["conv_post"] = (gen + M * d * 4 + 2 * M * d * 4, 2 * M * 2 * ng * d)
    return w


def step_bytes(dims, batch, ctx_lens, fp8=False):
    """Algorithmic HBM bytes of one whole step (weights once, KV once per layer, target logits)."""
    e = 2 if dims.dtype == "bf16" else 4
    d, H, Hkv, hd, F, V, L = dims.d, dims.n_heads, dims.n_kv_heads, dims.head_dim, dims.d_ffn, dims.vocab, dims.n_layers

    def wb(rows, cols):
        return rows * (cols + 16) if fp8 else rows * cols * e
    per_layer = wb((H + 2 * Hkv) * hd, d) + wb(d, H * hd) + wb(3 * F, d)
    conv = (4 * (2 * (d // 16) * d + 2 * d) * e) if dims.use_conv else 0
    weights = L * (per_layer + conv) + wb(V, d) + wb(d, dims.d_cat) + (3 * dims.ps_dim * d + 2 * dims.ps_rank * dims.ps_dim) * e
    kv = L * 2 * sum(ctx_lens) * Hkv * hd * e
    tgt = batch * 16 * V * e
    return weights + kv + tgt


# ------------------------------------------------------------------ CPU oracle baseline

def cpu_baseline(wl, W, seconds):
    """The oracle timed on this host's cores (BLAS on every core it may use), then again
    with BLAS held to one thread (half the time budget)."""
    from threadpoolctl import threadpool_info, threadpool_limits
    threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    allc = _cpu_run(wl, W, seconds, threads)
    with threadpool_limits(limits=1, user_api="blas"):
        one = _cpu_run(wl, W, seconds / 2, 1, warm_model=allc.pop("_model"))
    one.pop("_model", None)
    allc["one_thread"] = {k: one[k] for k in ("value", "unit", "cores", "sample")}
    return allc


def _cpu_run(wl, W, seconds, threads, warm_model=None):
    import numpy as np

    import oracle
    import synth
    dims = wl.dims
    L = int(wl.ctx_lens[0])
    cap = ((L + 16 + 31) // 32) * 32
    K, V = synth.make_cache(dims, [L], cap, wl.seed)
    kc = [oracle.decode(K[l, 0], dims.dtype) for l in range(dims.n_layers)]
    vc = [oracle.decode(V[l, 0], dims.dtype) for l in range(dims.n_layers)]
    hid = synth.make_hidden(dims, 16, wl.seed, key=2)
    ids = synth.make_block_ids(dims, 1, wl.seed, 1)[0]
    T = oracle.decode(synth.make_target_logits(dims, 1, 15, wl.seed, planted="random" if wl.planted else "none")[0],
                      dims.dtype)
    m = warm_model if warm_model is not None else oracle.Model(dims, W)
    pos = np.arange(L - 16, L) if L >= 16 else np.arange(0)
    t0 = time.perf_counter()
    oracle.drafting_step(m, kc, vc, L, hid[:len(pos)], pos, ids, T)        # warm-up: decodes the weights
    warm = time.perf_counter() - t0
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.drafting_step(m, kc, vc, L, hid[:len(pos)], pos, ids, T)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or (n >= 1 and el + el / n > 3 * seconds):
            break
    return {"value": n / el, "unit": "blocks/s", "cores": int(threads), "kind": "oracle",
            "host_cpus": len(os.sched_getaffinity(0)), "_model": m,
            "sample": f"{n} full drafting step(s) of sequence 0 (inject 16 rows, draft, path, verify) at the "
                      f"{wl.name} shapes, context {L}, float64 NumPy oracle on {threads} BLAS thread(s); "
                      f"{el:.1f} s timed after a {warm:.1f} s warm-up"}


# ------------------------------------------------------------------ main

def run_cycles(n, D, torch, np, synth, wl, dr, new_hid, row_off, tdt, log):
    """Full drafting cycles with the state on the device: inject n_new rows (the anchor and
    the accepted drafts of the previous cycle) at pos0, draft, choose the path, verify,
    advance, for every sequence of the workload, starting from its context lengths.  The
    cache is a second one with room for the growth (seeded noise of the injected rows'
    scale), so the timed step above keeps its own layout.  The target side is synthetic:
    its hidden rows are a fixed seeded buffer and its logits N(0,1) with +8 planted on the
    first A drafts and on another token at row A, A uniform in 0..15 per sequence and cycle
    (tau = 1 + E[A] = 8.5 by construction), planted by device tensor ops inside the timed
    loop.  Returns tau (mean emitted tokens per cycle) and tokens/s."""
    dims = wl.dims
    B, V = wl.batch, dims.vocab
    ctx = np.asarray(wl.ctx_lens, dtype=np.int32)
    warm = 3
    cap = ((int(ctx.max()) + 16 * (n + warm + 1) + 31) // 32) * 32
    dt_t = D.torch_dtype(dims)
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.seed + 4242)
    cache = D.KVCache(dims, B, cap, fill=None)
    scale = 0.02 * dims.d ** 0.5
    for l in range(dims.n_layers):
        for t in (cache.k[l], cache.vt[l]):
            t.copy_((torch.randn(t.shape, generator=g, device="cuda", dtype=torch.float32) * scale).to(dt_t))
    T0 = torch.randn((B, 16, V), generator=g, device="cuda", dtype=torch.float32).to(dt_t)
    T = torch.empty_like(T0)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()  # noqa: E731
    ctx_t = i32(ctx)
    pos0_t = i32(np.maximum(ctx - 16, 0))
    nnew_t = i32(np.minimum(ctx, 16))
    ids_t = i32(synth.make_block_ids(dims, B, wl.seed + 99, 1))
    ci = torch.zeros((B, 16, 16), dtype=torch.int32, device="cuda")
    cl = torch.zeros((B, 16, 16), dtype=torch.float32, device="cuda")
    fh = torch.zeros((B, 16, dims.d), dtype=torch.float32, device="cuda")
    pidx = torch.zeros((B, 15), dtype=torch.int32, device="cuda")
    pids = torch.zeros((B, 15), dtype=torch.int32, device="cuda")
    acc = torch.zeros(B, dtype=torch.int32, device="cuda")
    bon = torch.zeros(B, dtype=torch.int32, device="cuda")
    emitted = torch.zeros(B, dtype=torch.int64, device="cuda")
    rows = torch.arange(16, device="cuda")
    pad = torch.zeros((B, 1), dtype=torch.long, device="cuda")
    nb = {k: f for k, f in (("i", D.dflash_inject_workspace_bytes(dr.cfg, 16 * B)),
                            ("d", D.dflash_draft_workspace_bytes(dr.cfg, B, cap)),
                            ("p", D.dflash_path_workspace_bytes(dr.cfg, B)),
                            ("v", D.dflash_verify_workspace_bytes(B, 15, V)))}
    ws = {k: torch.empty(max(v, 256), dtype=torch.uint8, device="cuda") for k, v in nb.items()}

    def cycle():
        D.dflash_inject_context(dr.cfg, dr.w, cache.kv, new_hid, 16 * B, row_off, pos0_t, nnew_t, B,
                                ws["i"], nb["i"])
        D.dflash_draft_block(dr.cfg, dr.w, cache.kv, ctx_t, ids_t, B, ci, cl, fh, None, ws["d"], nb["d"])
        D.dflash_select_path(dr.cfg, dr.w, ci, cl, fh, ids_t, 1, D.DFLASH_PATH_GREEDY, B, pidx, pids, None,
                             ws["p"], nb["p"])
        # synthetic target: the first A drafts are its greedy tokens, row A holds another
        A = torch.randint(0, 16, (B, 1), generator=g, device="cuda")
        tok = torch.cat([pids.long(), pad], 1)
        other = (tok + 1 + torch.randint(0, V - 2, (B, 16), generator=g, device="cuda")) % (V - 1)
        T.copy_(T0)
        T.scatter_(2, torch.where(rows[None, :] < A, tok, other)[:, :, None], 8.0)
        D.dflash_verify(pids, T, tdt, B, 15, V, acc, bon, ws["v"], nb["v"])
        D.dflash_advance(acc, bon, B, dims.mask_id, cap, ctx_t, pos0_t, nnew_t, ids_t)
        emitted.add_(acc.long() + 1)

    for _ in range(warm):
        cycle()
    torch.cuda.synchronize()
    emitted.zero_()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(n):
        cycle()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / n
    tot = int(emitted.sum())
    tau = tot / (n * B)
    ctx_end = ctx_t.cpu().numpy()
    assert (ctx_end <= cap - 16).all(), "cycle cache overflow"
    tps = tot / (ms * n) * 1e3
    log(f"[bench] {n} cycles: {ms:.3f} ms/cycle, tau {tau:.2f}, {tps:.0f} tokens/s, "
        f"contexts now {ctx_end.min()}..{ctx_end.max()}")
    del cache
    return {"cycles": n, "ms_per_cycle": round(ms, 4), "tau": round(tau, 3), "tokens_per_s": round(tps, 1),
            "target": "synthetic: fixed seeded target hidden rows; target logits N(0,1) with +8 on the first A "
                      "drafts and on another token at row A, A ~ U{0..15} per sequence and cycle (tau = 8.5 "
                      "expected); planting by device tensor ops inside the timed loop"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the drafting step is built and "
              "measured on a single MI355X. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import block_diffusion_drafter_feature_amd as D
    import synth

    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    D.lib()
    wl = synth.workload(args.workload)
    dims = wl.dims
    B, cap = wl.batch, wl.cap
    ctx = np.asarray(wl.ctx_lens, dtype=np.int32)
    t0 = time.time()
    W = synth.make_weights(dims, wl.seed)
    dr = D.Drafter(dims, W)
    log(f"[bench] {wl.name}: weights {dr.nbytes() / 1e9:.2f} GB on device ({time.time() - t0:.1f} s)")
    if args.cpu_seconds <= 0:
        del W
        W = None
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()  # noqa: E731
    dt_t = D.torch_dtype(dims)

    # ---- prefill: inject every context row (device-generated N(0,1) target hiddens, one
    # chunk of at most 16384 rows per call), each call bracketed by events so that only the
    # injection itself is timed; or fill the cache directly (K after RoPE and V of an injected
    # row are ~N(0, 0.02^2 d) for unit-RMS context features).  The timed step reads the same
    # bytes either way.
    prefill = args.prefill
    cache = D.KVCache(dims, B, cap, fill=None if prefill == "synthetic" else 0.0)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.seed)
    t0 = time.time()
    prefill_info = None
    if prefill == "inject":
        chunk = 16384
        ws_inj = D.Workspace()
        marks, rows_done = [], 0
        pf_probe = D.Probes(("inject_fc", "inject_kv"))
        pieces = [(b, r0, min(chunk, int(ctx[b]) - r0)) for b in range(B) for r0 in range(0, int(ctx[b]), chunk)]
        # one untimed warm-up call (zero hiddens into the first piece's positions, which the
        # timed calls overwrite; the generator is not drawn from): the timed calls then run at
        # the steady clock
        warm = [pieces[0]] if pieces else []
        for i, (b, r0, n) in enumerate(warm + pieces):
            timed = i >= len(warm)
            if timed:
                hid = torch.randn((n, dims.d_cat), generator=gen, device="cuda", dtype=torch.float32).to(dt_t)
            else:
                hid = torch.zeros((n, dims.d_cat), device="cuda", dtype=dt_t)
            nb = D.dflash_inject_workspace_bytes(dr.cfg, n)
            sub = D.dflash_kv(batch=1, cap=cap)
            for l in range(dims.n_layers):
                sub.k[l] = cache.k[l][b].data_ptr()
                sub.vt[l] = cache.vt[l][b].data_ptr()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ws_buf = ws_inj.get(nb)
            e0.record()
            D.dflash_inject_context(dr.cfg, dr.w, sub, hid, n, i32([0, n]), i32([r0]), i32([n]), 1, ws_buf, nb,
                                    probes=pf_probe.struct if i == len(warm) + len(pieces) - 1 else None)
            e1.record()
            if timed:
                marks.append((e0, e1, n))
                rows_done += n
            del hid
        torch.cuda.synchronize()
        if marks:
            pf_ms = sum(a.elapsed_time(b_) for a, b_, _ in marks)
            kv_cols = dims.n_layers * 2 * dims.n_kv_heads * dims.head_dim
            flop_row = 2 * dims.d_cat * dims.d + 2 * dims.d * kv_cols
            tf = rows_done * flop_row / (pf_ms * 1e-3)
            n_last = marks[-1][2]
            fc_ms, kv_ms = pf_probe.ms("inject_fc"), pf_probe.ms("inject_kv")
            peak = MFMA_PEAK[dims.dtype]
            prefill_info = {
                "rows": rows_done, "calls": len(marks), "rows_per_call": chunk, "ms": round(pf_ms, 3),
                "rows_per_s": round(rows_done / (pf_ms * 1e-3), 1),
                "achieved": round(tf / 1e12, 1), "peak": peak / 1e12, "unit": "TFLOP/s", "frac": round(tf / peak, 4),
                "flop_per_row": int(flop_row),
                "last_call": {"rows": n_last,
                              "fusion_gemm": {"ms": round(fc_ms, 4), "frac": round(
                                  2 * n_last * dims.d_cat * dims.d / (fc_ms * 1e-3) / peak, 4)},
                              "kv_gemm": {"ms": round(kv_ms, 4), "frac": round(
                                  2 * n_last * dims.d * kv_cols / (kv_ms * 1e-3) / peak, 4)}},
                "includes": "per call: fusion GEMM, RMSNorm, K/V GEMM with RoPE and the cache scatter; the "
                            "target hiddens are generated outside the timed calls"}
            log(f"[bench] prefill injection: {rows_done} rows in {pf_ms:.1f} ms ({rows_done / pf_ms * 1e3:.0f} "
                f"rows/s, {tf / 1e12:.0f} TFLOP/s = {tf / peak:.3f} of peak)")
        del ws_inj
    else:
        scale = 0.02 * dims.d ** 0.5
        for l in range(dims.n_layers):
            for t in (cache.k[l], cache.vt[l]):
                t.copy_((torch.randn(t.shape, generator=gen, device="cuda", dtype=torch.float32) * scale).to(dt_t))
    torch.cuda.synchronize()
    log(f"[bench] prefill ({prefill}) of {int(ctx.sum())} context rows ({time.time() - t0:.1f} s)")

    # ---- step inputs (resident in HBM before timing)
    new_hid = D.to_device(synth.make_hidden(dims, 16 * B, wl.seed, key=2), dims)
    row_off = i32(np.arange(B + 1) * 16)
    pos0 = i32(np.maximum(ctx - 16, 0))
    n_new = i32(np.minimum(ctx, 16))
    ctx_t = i32(ctx)
    ids = synth.make_block_ids(dims, B, wl.seed, 1)
    ids_t = i32(ids)
    T = D.to_device(synth.make_target_logits(dims, B, 15, wl.seed, planted="random" if wl.planted else "none"), dims)
    tdt = D.DFLASH_BF16 if dims.dtype == "bf16" else D.DFLASH_F32
    ci = torch.zeros((B, 16, 16), dtype=torch.int32, device="cuda")
    cl = torch.zeros((B, 16, 16), dtype=torch.float32, device="cuda")
    fh = torch.zeros((B, 16, dims.d), dtype=torch.float32, device="cuda")
    pidx = torch.zeros((B, 15), dtype=torch.int32, device="cuda")
    pids = torch.zeros((B, 15), dtype=torch.int32, device="cuda")
    acc = torch.zeros(B, dtype=torch.int32, device="cuda")
    bon = torch.zeros(B, dtype=torch.int32, device="cuda")
    nb_i = D.dflash_inject_workspace_bytes(dr.cfg, 16 * B)
    nb_d = D.dflash_draft_workspace_bytes(dr.cfg, B, cap)
    nb_p = D.dflash_path_workspace_bytes(dr.cfg, B)
    nb_v = D.dflash_verify_workspace_bytes(B, 15, dims.vocab)
    ws_i, ws_d, ws_p, ws_v = (torch.empty(n, dtype=torch.uint8, device="cuda") for n in (nb_i, nb_d, nb_p, nb_v))

    def step(probes=None):
        D.dflash_inject_context(dr.cfg, dr.w, cache.kv, new_hid, 16 * B, row_off, pos0, n_new, B, ws_i, nb_i,
                                probes=probes.struct if probes else None)
        D.dflash_draft_block(dr.cfg, dr.w, cache.kv, ctx_t, ids_t, B, ci, cl, fh, None, ws_d, nb_d,
                             probes=probes.struct if probes else None)
        D.dflash_select_path(dr.cfg, dr.w, ci, cl, fh, ids_t, 1, D.DFLASH_PATH_GREEDY, B, pidx, pids, None,
                             ws_p, nb_p)
        D.dflash_verify(pids, T, tdt, B, 15, dims.vocab, acc, bon, ws_v, nb_v)

    # the library's streaming LM head (one drafted block, bf16) runs one work-group per
    # compute unit, each keeping its own top-16 lists (at most 256 of them)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    lists = min(cus, dims.vocab // 16) if (dims.dtype == "bf16" and B == 1 and dims.d == 4096
                                           and dims.vocab // 16 >= 384 and cus <= 256) else 0
    work = kernel_work(dims, B, wl.ctx_lens, lists=lists)
    # live kernel probes on every PROBE_EVERY-th timed step (each probe adds event records
    # to the stream, ~5 us apiece); the average is over the probed steps of the timed region
    probed = list(range(0, args.steps, PROBE_EVERY))
    live = {k: D.Probes(("lm_head", "attn")) for k in probed}
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for k in range(args.steps):
        step(live.get(k))
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    value = B * 1000.0 / ms
    log(f"[bench] {args.steps} steps: {ms:.3f} ms/step, {value:.1f} blocks/s")

    def avg_ms(probes, name):
        return float(np.mean([p.ms(name) for p in probes]))

    def roof(name, t_ms):
        by, fl = work[name]
        peak_mf = MFMA_PEAK[dims.dtype]
        bound = "mfma" if fl / max(by, 1) > peak_mf / HBM_PEAK else "hbm"
        if bound == "hbm":
            a = by / (t_ms * 1e-3)
            return {"bound": "hbm", "achieved": round(a / 1e9, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                    "frac": round(a / HBM_PEAK, 4), "algorithmic_bytes": int(by), "ms": round(t_ms, 4)}
        a = fl / (t_ms * 1e-3)
        return {"bound": "mfma", "achieved": round(a / 1e12, 1), "peak": peak_mf / 1e12, "unit": "TFLOP/s",
                "frac": round(a / peak_mf, 4), "algorithmic_flops": int(fl), "ms": round(t_ms, 4)}

    # the dominant kernel: the larger share of the step's time, the LM head (one launch per
    # step) or the block attention (one launch per layer)
    lm_ms, at_ms = avg_ms(live.values(), "lm_head"), avg_ms(live.values(), "attn")
    dominant = "attn" if at_ms * dims.n_layers > lm_ms else "lm_head"
    dom = roof(dominant, lm_ms if dominant == "lm_head" else at_ms)
    attn = roof("attn", at_ms)
    lmh = roof("lm_head", lm_ms)
    traffic = None
    tpath = os.path.join(ROOT, "profiles", f"traffic_{wl.name}.json")
    if os.path.exists(tpath):
        try:
            import hashlib
            tr = json.load(open(tpath))
            tr = tr.get(dominant, tr)   # one entry per kernel, or a single kernel's entry
            src = hashlib.sha256(open(os.path.join(ROOT, "block_diffusion_drafter_feature_amd", "csrc",
                                                   tr["source"]), "rb").read()).hexdigest()
            if tr.get("kernel") == dominant and tr.get("source_sha256") == src:
                traffic = tr["bytes_per_launch"]
        except Exception:
            traffic = None
    roofline = {k: dom[k] for k in ("bound", "achieved", "peak", "unit", "frac")}
    kname = ("gemm_skinny_kernel" if dims.dtype != "bf16" else
             "gemm_stream_kernel" if wl.batch == 1 else "gemm_pipe_kernel")
    epi = "EpiLogitsTop16" if lists else "EpiLogits"
    kdesc = (f"lm_head GEMM ({kname}<..., {epi}>)" if dominant == "lm_head" else
             "block attention, one layer (block_attn_kernel + attn_combine_kernel)")
    roofline.update({"traffic": traffic, "kernel": kdesc, "share_of_step": round(
                         (lm_ms if dominant == "lm_head" else at_ms * dims.n_layers) / ms, 4),
                     "algorithmic_bytes_per_launch": dom.get("algorithmic_bytes"), "ms_per_launch": dom["ms"]})

    breakdown = {}
    if not args.no_breakdown:
        names = ["lm_head", "topk", "attn", "qkv", "o", "gate_up", "down", "inject_fc", "inject_kv"]
        if dims.use_conv:
            names += ["conv_pre", "conv_post"]
        pr = [D.Probes(tuple(names)) for _ in range(5)]
        for p in pr:
            step(p)
        torch.cuda.synchronize()
        for n in names:
            breakdown[n] = roof(n, avg_ms(pr, n)) if n != "topk" else {"ms": round(avg_ms(pr, n), 4)}

    # the same step captured once in a HIP graph and replayed (what a serving loop that
    # cannot afford per-kernel launches would run); reported apart, never as the value
    graph = None
    if args.graph_steps > 0:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            step()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.graph_steps):
            g.replay()
        stop.record()
        torch.cuda.synchronize()
        ms_g = start.elapsed_time(stop) / args.graph_steps
        log(f"[bench] graph replays: {ms_g:.3f} ms/step, {B * 1000.0 / ms_g:.1f} blocks/s")
        graph = {"steps": args.graph_steps, "ms_per_step": round(ms_g, 4), "blocks_per_s": round(B * 1000.0 / ms_g, 2),
                 "what": "inject, draft, greedy path and verify captured once in a HIP graph, replayed"}
        del g

    sampled = None
    if args.sampled_steps > 0:
        temp = 0.8
        rng = torch.Generator(device="cuda")
        rng.manual_seed(wl.seed + 77)
        u_path = torch.rand((B, 15), generator=rng, device="cuda")
        u_acc = torch.rand((B, 15), generator=rng, device="cuda")
        u_bon = torch.rand((B,), generator=rng, device="cuda")
        pq = torch.zeros((B, 15, 16), dtype=torch.float32, device="cuda")
        nb_s = D.dflash_verify_sampled_workspace_bytes(B, 15, dims.vocab)
        ws_s = torch.empty(nb_s, dtype=torch.uint8, device="cuda")
        cand_rows = ci[:, 1:].data_ptr()          # rows 1..15 of the draft call's candidates

        def sampled_step():
            D.dflash_inject_context(dr.cfg, dr.w, cache.kv, new_hid, 16 * B, row_off, pos0, n_new, B, ws_i, nb_i)
            D.dflash_draft_block(dr.cfg, dr.w, cache.kv, ctx_t, ids_t, B, ci, cl, fh, None, ws_d, nb_d)
            D.dflash_sample_path(dr.cfg, dr.w, ci, cl, fh, ids_t, 1, B, temp, u_path, pidx, pids, pq, None,
                                 ws_p, nb_p)
            D.dflash_verify_sampled(pids, cand_rows, 256, pq, T, tdt, B, 15, dims.vocab, temp, u_acc, u_bon, acc,
                                    bon, ws_s, nb_s)

        for _ in range(3):
            sampled_step()
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.sampled_steps):
            sampled_step()
        stop.record()
        torch.cuda.synchronize()
        ms_s = start.elapsed_time(stop) / args.sampled_steps
        log(f"[bench] sampling variant: {ms_s:.3f} ms/step, {B * 1000.0 / ms_s:.1f} blocks/s")
        sampled = {"steps": args.sampled_steps, "ms_per_step": round(ms_s, 4),
                   "blocks_per_s": round(B * 1000.0 / ms_s, 2), "temperature": temp,
                   "path": "sampled over the pair scores", "verify": "rejection sampling"}

    fp8 = None
    if args.fp8_steps > 0 and dims.dtype == "bf16":
        dr8 = D.Drafter(dims, dr.t, fp8=True)       # quantized on the device from the bf16 copies

        def step8(probes=None):
            D.dflash_inject_context(dr8.cfg, dr8.w, cache.kv, new_hid, 16 * B, row_off, pos0, n_new, B, ws_i, nb_i,
                                    probes=probes.struct if probes else None)
            D.dflash_draft_block(dr8.cfg, dr8.w, cache.kv, ctx_t, ids_t, B, ci, cl, fh, None, ws_d, nb_d,
                                 probes=probes.struct if probes else None)
            D.dflash_select_path(dr8.cfg, dr8.w, ci, cl, fh, ids_t, 1, D.DFLASH_PATH_GREEDY, B, pidx, pids, None,
                                 ws_p, nb_p)
            D.dflash_verify(pids, T, tdt, B, 15, dims.vocab, acc, bon, ws_v, nb_v)

        live8 = {k: D.Probes(("lm_head", "attn")) for k in range(0, args.fp8_steps, PROBE_EVERY)}
        for _ in range(3):
            step8()
        torch.cuda.synchronize()
        start.record()
        for k in range(args.fp8_steps):
            step8(live8.get(k))
        stop.record()
        torch.cuda.synchronize()
        ms8 = start.elapsed_time(stop) / args.fp8_steps
        w8 = kernel_work(dims, B, wl.ctx_lens, fp8=True, lists=lists)
        lm_ms = float(np.mean([p.ms("lm_head") for p in live8.values()]))
        lm_bytes = w8["lm_head"][0]
        sb8 = step_bytes(dims, B, wl.ctx_lens, fp8=True)
        log(f"[bench] fp8 weights: {ms8:.3f} ms/step, {B * 1000.0 / ms8:.1f} blocks/s, LM head {lm_ms * 1e3:.1f} us")
        fp8 = {"steps": args.fp8_steps, "ms_per_step": round(ms8, 4), "blocks_per_s": round(B * 1000.0 / ms8, 2),
               "weights": "E4M3 codes + float32 scale per row for the streamed projections; bf16 activations and "
                          "bf16 matrix-core products (codes widened exactly), fp32 accumulation",
               "lm_head": {"bound": "hbm", "achieved": round(lm_bytes / (lm_ms * 1e-3) / 1e9, 1),
                           "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                           "frac": round(lm_bytes / (lm_ms * 1e-3) / HBM_PEAK, 4),
                           "algorithmic_bytes_per_launch": int(lm_bytes), "ms_per_launch": round(lm_ms, 4)},
               "step_roofline": {"algorithmic_bytes": int(sb8), "hbm_bound_ms": round(sb8 / HBM_PEAK * 1e3, 4),
                                 "frac": round(sb8 / HBM_PEAK * 1e3 / ms8, 4)},
               "weight_bytes_on_device": int(dr8.nbytes())}
        del dr8

    smaller = {}
    for bs in [int(x) for x in args.block_sizes.split(",") if x.strip()]:
        if not 2 <= bs <= 16:
            continue
        drb = D.Drafter(dims, dr.t, block_size=bs)
        Tb = T[:, :bs].contiguous()
        nb_vb = D.dflash_verify_workspace_bytes(B, bs - 1, dims.vocab)
        ws_vb = torch.empty(nb_vb, dtype=torch.uint8, device="cuda")
        idx_b = torch.zeros((B, bs - 1), dtype=torch.int32, device="cuda")
        ids_b = torch.zeros((B, bs - 1), dtype=torch.int32, device="cuda")

        def step_b():
            D.dflash_inject_context(drb.cfg, drb.w, cache.kv, new_hid, 16 * B, row_off, pos0, n_new, B, ws_i, nb_i)
            D.dflash_draft_block(drb.cfg, drb.w, cache.kv, ctx_t, ids_t, B, ci, cl, fh, None, ws_d, nb_d)
            D.dflash_select_path(drb.cfg, drb.w, ci, cl, fh, ids_t, 1, D.DFLASH_PATH_GREEDY, B, idx_b, ids_b, None,
                                 ws_p, nb_p)
            D.dflash_verify(ids_b, Tb, tdt, B, bs - 1, dims.vocab, acc, bon, ws_vb, nb_vb)

        for _ in range(3):
            step_b()
        torch.cuda.synchronize()
        nsteps = max(1, args.steps // 2)
        start.record()
        for _ in range(nsteps):
            step_b()
        stop.record()
        torch.cuda.synchronize()
        msb = start.elapsed_time(stop) / nsteps
        log(f"[bench] block size {bs}: {msb:.3f} ms/step")
        smaller[str(bs)] = {"steps": nsteps, "ms_per_step": round(msb, 4), "blocks_per_s": round(B * 1000.0 / msb, 2)}
        del drb

    calib = None
    if args.cal_dim > 0:
        C, V, d = args.cal_dim, dims.vocab, dims.d
        gcal = torch.Generator(device="cuda")
        gcal.manual_seed(wl.seed + 31)
        cw = {"cal_w1": (torch.randn((C, 2 * d), generator=gcal, device="cuda") * 0.02).to(dt_t),
              "cal_w2": (torch.randn((V, C), generator=gcal, device="cuda") * 0.02).to(dt_t)}
        drc = D.Drafter(dims, {**dr.t, **cw})
        lg_full = torch.zeros((B, 16, V), dtype=torch.float32, device="cuda")
        D.dflash_draft_block(dr.cfg, dr.w, cache.kv, ctx_t, ids_t, B, ci, cl, fh, lg_full, ws_d, nb_d)
        nb_c = D.dflash_calibrate_workspace_bytes(drc.cfg, B)
        ws_c = torch.empty(nb_c, dtype=torch.uint8, device="cuda")
        ci_c = torch.zeros_like(ci)
        cl_c = torch.zeros_like(cl)
        for _ in range(3):
            D.dflash_calibrate(drc.cfg, drc.w, fh, bon, B, lg_full, ci_c, cl_c, ws_c, nb_c)
        torch.cuda.synchronize()
        ncal = max(10, args.steps)
        start.record()
        for _ in range(ncal):
            D.dflash_calibrate(drc.cfg, drc.w, fh, bon, B, lg_full, ci_c, cl_c, ws_c, nb_c)
        stop.record()
        torch.cuda.synchronize()
        msc = start.elapsed_time(stop) / ncal
        e = 2 if dims.dtype == "bf16" else 4
        M = 16 * B
        cal_bytes = V * C * e + C * 2 * d * e + M * 2 * d * e + 3 * M * V * 4
        log(f"[bench] calibration (width {C}): {msc * 1e3:.1f} us per block batch")
        calib = {"calls": ncal, "ms_per_call": round(msc, 4), "cal_dim": C,
                 "algorithmic_bytes": int(cal_bytes),
                 "hbm_frac": round(cal_bytes / (msc * 1e-3) / HBM_PEAK, 4),
                 "includes": "input gather, MLP input GEMM (SiLU), output GEMM adding into the logits, top-16"}
        del drc, cw

    cycle = None
    if args.cycles > 0:
        cycle = run_cycles(args.cycles, D, torch, np, synth, wl, dr, new_hid, row_off, tdt, log)

    if args.copy_mib > 0:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.randn(n, device="cuda", dtype=torch.float32)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: {n * 4} bytes read and {n * 4} bytes written per launch, 3 launches")
        del src, dst

    cpu = None
    if W is not None:
        log(f"[bench] CPU oracle sample ({args.cpu_seconds:.0f} s budget) ...")
        cpu = cpu_baseline(wl, W, args.cpu_seconds)
        log(f"[bench] CPU oracle: {cpu['value']:.4f} blocks/s on {cpu['cores']} BLAS threads, "
            f"{cpu['one_thread']['value']:.4f} on one")

    sb = step_bytes(dims, B, wl.ctx_lens)
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "blocks/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dims.dtype, "data": "synthetic (seeded random-init weights, N(0,1) hiddens/logits)",
        "config": {"workload": f"{wl.name}: {wl.description}", "batch": B,
                   "context": list(map(int, wl.ctx_lens)) if B <= 4 else {"min": int(ctx.min()), "max": int(ctx.max()),
                                                                          "sum": int(ctx.sum())},
                   "block": 16, "d_model": dims.d, "heads": f"{dims.n_heads}q/{dims.n_kv_heads}kv x {dims.head_dim}",
                   "d_ffn": dims.d_ffn, "layers": dims.n_layers, "fusion": f"{dims.d_cat}->{dims.d}",
                   "vocab": dims.vocab, "topk": 16, "conv": bool(dims.use_conv), "gate": bool(dims.use_gate),
                   "path": "greedy", "prefill": prefill, "parallelism": "single GPU"},
        "roofline": roofline,
        "attention": {k: attn[k] for k in ("bound", "achieved", "peak", "unit", "frac", "ms")},
        "lm_head": {k: lmh[k] for k in ("bound", "achieved", "peak", "unit", "frac", "ms")},
        "prefill": prefill_info,
        "step_roofline": {"algorithmic_bytes": int(sb), "hbm_bound_ms": round(sb / HBM_PEAK * 1e3, 4),
                          "frac": round(sb / HBM_PEAK * 1e3 / ms, 4)},
        "breakdown": breakdown,
        "cpu_baseline": cpu,
    }
    if graph is not None:
        out["graph"] = graph
    if sampled is not None:
        out["sampled"] = sampled
    if fp8 is not None:
        out["fp8_weights"] = fp8
    if smaller:
        out["smaller_blocks"] = smaller
    if calib is not None:
        out["calibration"] = calib
    if cycle is not None:
        out["cycle"] = cycle
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
