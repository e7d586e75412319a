"""Shared helpers of the GPU parity tests: tolerances, comparisons, oracle batch runs."""
import numpy as np

import oracle

# Tolerance on continuous outputs (hidden states, logits, scores, cache rows): per row,
# ||gpu - oracle||_inf / ||oracle||_inf.  bf16 workloads: 2e-2 (bf16 operands, fp32
# accumulation; the oracle keeps fp64 between the bf16 contract points, so a bf16
# rounding that lands on the other side of a tie is one bf16 ulp, 2^-8, of one
# element, and the fp32 accumulation adds ~1e-6).  fp32 workloads: 1e-4.
def tol(dims) -> float:
    return 2e-2 if dims.dtype == "bf16" else 1e-4


def tol_conditioned(dims, kappa: float) -> float:
    """The stated tolerance, or three times the computation's own fp32-level spread on the
    inputs at hand (``conditioning``) where that is larger: no fp32 implementation can be
    held closer to an fp64 oracle than the oracle's own result moves under fp32 noise."""
    return max(tol(dims), 3.0 * kappa)


def rowwise_relerr(g: np.ndarray, o: np.ndarray) -> float:
    g = np.asarray(g, dtype=np.float64).reshape(-1, np.shape(g)[-1])
    o = np.asarray(o, dtype=np.float64).reshape(-1, np.shape(o)[-1])
    num = np.abs(g - o).max(axis=1)
    den = np.maximum(np.abs(o).max(axis=1), 1e-30)
    return float((num / den).max()) if len(num) else 0.0


def assert_close_rows(name, g, o, t):
    assert np.isfinite(np.asarray(g, dtype=np.float64)).all(), f"{name}: non-finite GPU values"
    e = rowwise_relerr(g, o)
    assert e <= t, f"{name}: row-wise max relative error {e:.3e} > {t:.1e}"
    return e


def topk_with_margin(gpu_ids, oracle_logits, gpu_logits, k=16):
    """Check GPU top-k ids against the oracle's logits.

    Where the oracle's ranking is decided by more than twice the row's observed error,
    the ids must be equal; a swap is accepted only between entries whose oracle logits are
    within that margin.  Returns the number of accepted near-tie differences."""
    lo = np.asarray(oracle_logits, dtype=np.float64)
    lg = np.asarray(gpu_logits, dtype=np.float64)
    oi, _ = oracle.topk(lo, k)
    gi = np.asarray(gpu_ids)
    diffs = 0
    for r in range(lo.shape[0]):
        margin = 2.0 * np.abs(lg[r] - lo[r]).max() + 1e-12
        if np.array_equal(gi[r], oi[r]):
            continue
        for kk in range(k):
            if gi[r, kk] != oi[r, kk]:
                assert abs(lo[r, gi[r, kk]] - lo[r, oi[r, kk]]) <= margin, (
                    f"row {r} rank {kk}: gpu id {gi[r, kk]} vs oracle id {oi[r, kk]}, "
                    f"oracle gap {abs(lo[r, gi[r, kk]] - lo[r, oi[r, kk]]):.3e} > margin {margin:.3e}")
                diffs += 1
    return diffs


def exact_topk_of(logits: np.ndarray, k=16):
    """Top-k ids of given logits by a stable full sort (value desc, id asc)."""
    lg = np.asarray(logits, dtype=np.float32)
    ids = np.empty(lg.shape[:-1] + (k,), dtype=np.int32)
    flat = lg.reshape(-1, lg.shape[-1])
    for r in range(flat.shape[0]):
        ids.reshape(-1, k)[r] = np.lexsort((np.arange(flat.shape[1]), -flat[r].astype(np.float64)))[:k]
    return ids


def walk_f32(cand_logits, S, has_anchor, mode):
    """The path walk over given fp32 scores, in fp32 and in the summation order the device
    documents (used to check that a device path is the walk of its own scores)."""
    lg = np.asarray(cand_logits, dtype=np.float32)
    S = np.asarray(S, dtype=np.float32)
    P = lg.shape[0]
    first = lg[0] + (S[0, 0] if has_anchor else np.float32(0))
    if mode == "greedy":
        idx = [int(np.argmax(first))]
        for p in range(1, P):
            idx.append(int(np.argmax(lg[p] + S[p, idx[-1]])))
        return np.asarray(idx)
    best = first.astype(np.float32)
    back = np.zeros((P, 16), dtype=np.int64)
    for p in range(1, P):
        cand = best[:, None] + S[p]
        back[p] = np.argmax(cand, axis=0)
        best = lg[p] + cand[back[p], np.arange(16)]
    j = int(np.argmax(best))
    idx = [j]
    for p in range(P - 1, 0, -1):
        j = int(back[p, j])
        idx.append(j)
    return np.asarray(idx[::-1])


def accept_of(draft, target_logits):
    """Accepted length and bonus token of a device draft under given target logits, by
    direct inspection (largest logit, lowest id on ties): a validity check of device
    outputs, independent of the oracle module."""
    t = np.asarray(target_logits, dtype=np.float64)
    greedy = [int(np.flatnonzero(row == row.max())[0]) for row in t]
    a = 0
    while a < len(draft) and int(draft[a]) == greedy[a]:
        a += 1
    return a, greedy[a]


def conditioning(m, kc, vc, ctx_len, block_ids, base, seeds=(0, 1)):
    """How far the oracle's own result moves when every value is perturbed by about one
    fp32 ulp (relative 2^-24, random sign) just before each bf16 rounding point: the
    spread that fp32 arithmetic alone can produce on these inputs.  Returns the row-wise
    relative deviation (max over logits and final hidden, max over seeds)."""
    worst = 0.0
    for sd in seeds:
        r = np.random.default_rng(sd)

        class Perturbed(oracle.Model):
            def rb(self, x):
                x = np.asarray(x, dtype=np.float64)
                if self.dims.dtype != "bf16":
                    return x
                return oracle.bf16_round(x * (1 + r.uniform(-2.0 ** -24, 2.0 ** -24, size=x.shape)))

        mp = Perturbed(m.dims, m.stored)
        mp._cache = m._cache
        o = oracle.draft_block(mp, kc, vc, ctx_len, block_ids)
        worst = max(worst, rowwise_relerr(o["logits"], base["logits"]), rowwise_relerr(o["xhat"], base["xhat"]))
    return worst


def oracle_draft(m, K, V, ctx_lens, block_ids):
    """Oracle draft of every sequence: K, V logical caches [L][B][Hkv][cap][hd] stored arrays."""
    D = m.dims
    outs = []
    for b, L in enumerate(ctx_lens):
        kc = [oracle.decode(K[l, b], D.dtype) for l in range(D.n_layers)]
        vc = [oracle.decode(V[l, b], D.dtype) for l in range(D.n_layers)]
        outs.append(oracle.draft_block(m, kc, vc, int(L), block_ids[b]))
    return outs


def draw_f32(q, u):
    """The device's inverse-CDF draw over given fp32 probabilities, in its documented
    order: total and running sum sequential in fp32, target = u * total; the first index
    whose running sum exceeds the target, else the last index of positive probability."""
    q = np.asarray(q, dtype=np.float32)
    tot = np.float32(0)
    for v in q:
        tot = np.float32(tot + v)
    target = np.float32(np.float32(u) * tot)
    run = np.float32(0)
    for i, v in enumerate(q):
        run = np.float32(run + v)
        if target < run:
            return i
    return int(np.flatnonzero(q > 0)[-1])
