"""Parity of the sampled path choice and of verification by rejection sampling.

Both take their uniforms as inputs, so the device and the oracle make the same draws.
Discrete results are compared exactly where both sides decide on the same numbers (the
device's draw over its own probabilities), and against the oracle's float64 decisions
up to near ties: a difference is accepted only where the uniform lies within the
observed floating-point error of a decision boundary.  A statistical check on the
device shows the property that defines rejection sampling: whatever the proposal, the
emitted token is distributed as the target's softmax.
"""
import sys

import numpy as np
import pytest
from scipy.special import softmax
from scipy.stats import chi2

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


def f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def ws_of(n):
    return torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")


class Ns:
    def __init__(self, **kw):
        self.__dict__.update(kw)


# ------------------------------------------------------------------ sampled path choice

SAMPLE_CASES = [("t_small", 1, 1.0), ("t_small", 0, 0.7), ("t_conv", 1, 1.5), ("t_f32", 1, 1.0), ("t_f32", 0, 0.5),
                ("c1", 1, 0.8)]


@pytest.mark.parametrize("name,n_fixed,temp", SAMPLE_CASES)
def test_sample_path_parity(name, n_fixed, temp):
    say(f"sample path {name} n_fixed={n_fixed} t={temp}")
    wl = synth.workload(name)
    dims = wl.dims
    B = max(wl.batch, 6)
    W = synth.make_weights(dims, wl.seed, ps_scale="stress")
    ids, lg, xh = synth.make_candidates(dims, B, wl.seed + 1)
    bids = synth.make_block_ids(dims, B, wl.seed + 1, n_fixed)
    P = 16 - n_fixed
    u = np.random.default_rng(wl.seed + 2).uniform(size=(B, P)).astype(np.float32)
    dr = D.Drafter(dims, W)
    pidx = torch.zeros((B, P), dtype=torch.int32, device="cuda")
    pids = torch.zeros((B, P), dtype=torch.int32, device="cuda")
    pq = torch.zeros((B, P, 16), dtype=torch.float32, device="cuda")
    ps = torch.zeros((B, P, 16, 16), dtype=torch.float32, device="cuda")
    nb = D.dflash_path_workspace_bytes(dr.cfg, B)
    D.dflash_sample_path(dr.cfg, dr.w, i32(ids), f32(lg), f32(xh), i32(bids), n_fixed, B, temp, f32(u), pidx, pids,
                         pq, ps, ws_of(nb), nb)
    torch.cuda.synchronize()
    pidx, pids, pq, ps = (x.cpu().numpy() for x in (pidx, pids, pq, ps))
    m = oracle.Model(dims, W)
    t = H.tol(dims)
    near = 0
    for b in range(B):
        S = oracle.path_pair_scores(m, ids[b], xh[b], bids[b], n_fixed)
        H.assert_close_rows(f"pair scores b{b}", ps[b].reshape(-1, 16), S.reshape(-1, 16), t)
        lgb = lg[b, n_fixed:].astype(np.float64)
        np.testing.assert_array_equal(pids[b], ids[b, n_fixed:][np.arange(P), pidx[b]])
        # the device's probabilities are the softmax of its own scores along its own path,
        # and its draw inverts them exactly as documented
        for p in range(P):
            prev = pidx[b][p - 1] if p > 0 else 0
            sc = lgb[p] + (ps[b][p, prev] if (p > 0 or n_fixed) else 0.0)
            np.testing.assert_allclose(pq[b, p], softmax(sc / temp), atol=1e-5, rtol=0)
            assert pidx[b][p] == H.draw_f32(pq[b, p], u[b, p]), (b, p)
        # against the oracle's own scores and draws: equal up to the first near tie
        oidx, oq = oracle.sample_path(lgb, S, n_fixed == 1, temp, u[b].astype(np.float64))
        for p in range(P):
            prev = pidx[b][p - 1] if p > 0 else 0
            scd = lgb[p] + (ps[b][p, prev] if (p > 0 or n_fixed) else 0.0)
            sco = lgb[p] + (S[p, prev] if (p > 0 or n_fixed) else 0.0)
            delta = np.abs(scd - sco).max()
            bound = (np.exp(2 * delta / temp) - 1) * oq[p].max() + 1e-6
            assert np.abs(pq[b, p] - oq[p]).max() <= bound, (b, p, np.abs(pq[b, p] - oq[p]).max(), bound)
            if oidx[p] != pidx[b][p]:
                cum = np.cumsum(oq[p])
                lo, hi = sorted((int(oidx[p]), int(pidx[b][p])))
                gap = min(abs(float(u[b, p]) - cum[k]) for k in range(lo, hi))
                assert gap <= 16 * bound, (b, p, gap, bound)
                near += 1
                break
    say(f"  near-tie draw differences: {near}")


# ------------------------------------------------------------------ rejection sampling

def make_proposals(V, B, P, seed, conc=0.5):
    """Sparse proposals (16 distinct ids, Dirichlet probabilities) and drafts drawn from them."""
    r = np.random.default_rng(seed)
    q_ids = np.zeros((B, P, 16), dtype=np.int32)
    q_probs = np.zeros((B, P, 16), dtype=np.float32)
    draft = np.zeros((B, P), dtype=np.int32)
    for b in range(B):
        for i in range(P):
            q_ids[b, i] = r.choice(V - 1, size=16, replace=False)
            qp = r.dirichlet(np.full(16, conc)).astype(np.float32)
            q_probs[b, i] = qp
            draft[b, i] = q_ids[b, i][r.choice(16, p=qp.astype(np.float64) / qp.astype(np.float64).sum())]
    return q_ids, q_probs, draft


def check_against_oracle(T, q_ids, q_probs, draft, temp, ua, ub, acc, bon, tag):
    """Device (a, bonus) per sequence against the oracle, up to near ties."""
    B, P = draft.shape
    near = 0
    for b in range(B):
        a_o, b_o = oracle.verify_sampled(draft[b], q_ids[b], q_probs[b].astype(np.float64), T[b], temp,
                                         ua[b].astype(np.float64), float(ub[b]))
        if (a_o, b_o) == (int(acc[b]), int(bon[b])):
            continue
        Tb = T[b].astype(np.float64)
        probs = [softmax(Tb[i] / temp) for i in range(P + 1)]
        if a_o != int(acc[b]):
            i = min(a_o, int(acc[b]))
            x = int(draft[b, i])
            hit = np.flatnonzero(q_ids[b, i] == x)
            q = float(q_probs[b, i][hit[0]])
            rel = abs(float(ua[b, i]) * q - probs[i][x]) / max(probs[i][x], 1e-30)
            assert rel < 1e-4, f"{tag} b{b}: accept {acc[b]} vs oracle {a_o}, margin {rel:.2e}"
        else:
            a = a_o
            r = probs[a].copy()
            if a < P:
                r[q_ids[b, a]] = np.maximum(0.0, r[q_ids[b, a]] - q_probs[b, a])
            cum = np.cumsum(r)
            target = float(ub[b]) * cum[-1]
            lo, hi = sorted((b_o, int(bon[b])))
            gap = min(abs(target - cum[k]) for k in range(lo, hi))
            assert gap < 1e-4 * cum[-1], f"{tag} b{b}: bonus {bon[b]} vs oracle {b_o}, gap {gap:.2e}"
        near += 1
    return near


VS_CASES = [
    # B, P, V, dtype, temperature, boost, seed
    (8, 15, 1024, "f32", 1.0, 8.0, 31),
    (8, 15, 1024, "bf16", 0.7, 6.0, 32),
    (5, 7, 4099, "f32", 1.3, 10.0, 33),
    (3, 0, 3000, "bf16", 1.0, 0.0, 34),
    (4, 64, 512, "f32", 1.0, 9.0, 35),
    (32, 15, 151936, "bf16", 0.6, 9.0, 36),
]


@pytest.mark.parametrize("B,P,V,dt,temp,boost,seed", VS_CASES)
def test_verify_sampled_parity(B, P, V, dt, temp, boost, seed):
    say(f"verify_sampled B={B} P={P} V={V} {dt} t={temp}")
    dims = Ns(vocab=V, dtype=dt)
    q_ids, q_probs, draft = make_proposals(V, B, P, seed)
    Tst = synth.make_target_logits(dims, B, P, seed, planted="prefix" if P else "none", draft=draft if P else None,
                                   boost=boost)
    T = synth.bits_to_f32(Tst) if dt == "bf16" else Tst
    r = np.random.default_rng(seed + 1)
    ua = r.uniform(size=(B, P)).astype(np.float32)
    ub = r.uniform(size=B).astype(np.float32)
    Td = torch.from_numpy(Tst.view(np.int16) if dt == "bf16" else Tst).cuda()
    if dt == "bf16":
        Td = Td.view(torch.bfloat16)
    acc = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    bon = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    nb = D.dflash_verify_sampled_workspace_bytes(B, P, V)
    tdt = D.DFLASH_BF16 if dt == "bf16" else D.DFLASH_F32
    D.dflash_verify_sampled(i32(draft) if P else None, i32(q_ids) if P else None, 16 * P, f32(q_probs) if P else None,
                            Td, tdt, B, P, V, temp, f32(ua) if P else None, f32(ub), acc, bon, ws_of(nb), nb)
    torch.cuda.synchronize()
    acc, bon = acc.cpu().numpy(), bon.cpu().numpy()
    assert ((acc >= 0) & (acc <= P)).all() and ((bon >= 0) & (bon < V)).all()
    near = check_against_oracle(T, q_ids, q_probs, draft, temp, ua, ub, acc, bon, f"V={V}")
    say(f"  accept lengths {acc.tolist()[:12]}, near ties {near}")
    assert near <= max(1, B // 8)


def test_verify_sampled_reads_the_draft_calls_candidate_layout():
    """q_ids given as the draft call's [B, 16, 16] candidate array offset by one row, with
    a stride of 256, gives the same result as a dense copy."""
    B, P, V, temp = 6, 15, 2048, 0.9
    q_ids, q_probs, draft = make_proposals(V, B, P, 41)
    full = np.zeros((B, 16, 16), dtype=np.int32)
    full[:, 0] = 7
    full[:, 1:] = q_ids
    T = synth.make_target_logits(Ns(vocab=V, dtype="f32"), B, P, 41, planted="prefix", draft=draft, boost=9.0)
    r = np.random.default_rng(42)
    ua, ub = r.uniform(size=(B, P)).astype(np.float32), r.uniform(size=B).astype(np.float32)
    nb = D.dflash_verify_sampled_workspace_bytes(B, P, V)
    outs = []
    for qi, stride in ((i32(q_ids), 16 * P), (i32(full)[:, 1:], 256)):
        acc = torch.zeros(B, dtype=torch.int32, device="cuda")
        bon = torch.zeros(B, dtype=torch.int32, device="cuda")
        D.dflash_verify_sampled(i32(draft), qi.data_ptr(), stride, f32(q_probs), f32(T), D.DFLASH_F32, B, P, V, temp,
                                f32(ua), f32(ub), acc, bon, ws_of(nb), nb)
        torch.cuda.synchronize()
        outs.append((acc.cpu().numpy(), bon.cpu().numpy()))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_rejection_sampling_is_lossless_on_device(dt):
    """16384 sequences share one target row and one proposal; each draws its draft from the
    proposal.  The first emitted token (the draft if accepted, else the bonus) must follow
    the target's softmax: chi-square over the tokens, seeded (deterministic)."""
    B, P, V, temp = 16384, 1, 64, 0.8
    r = np.random.default_rng(51)
    T0 = (r.standard_normal((P + 1, V)) * 1.5).astype(np.float32)
    if dt == "bf16":
        T0 = synth.bits_to_f32(synth.f32_to_bf16_bits(T0))
    ids = r.choice(V, size=16, replace=False).astype(np.int32)
    qp = r.dirichlet(np.full(16, 0.4)).astype(np.float32)
    draft = ids[r.choice(16, size=(B, P), p=qp.astype(np.float64) / qp.astype(np.float64).sum())]
    ua, ub = r.uniform(size=(B, P)).astype(np.float32), r.uniform(size=B).astype(np.float32)
    T = np.broadcast_to(T0, (B, P + 1, V)).copy()
    Td = torch.from_numpy(T).cuda()
    if dt == "bf16":
        Td = Td.to(torch.bfloat16)
    acc = torch.zeros(B, dtype=torch.int32, device="cuda")
    bon = torch.zeros(B, dtype=torch.int32, device="cuda")
    nb = D.dflash_verify_sampled_workspace_bytes(B, P, V)
    D.dflash_verify_sampled(i32(draft), i32(np.broadcast_to(ids, (B, P, 16))), 16 * P,
                            f32(np.broadcast_to(qp, (B, P, 16))), Td, D.DFLASH_BF16 if dt == "bf16" else D.DFLASH_F32,
                            B, P, V, temp, f32(ua), f32(ub), acc, bon, ws_of(nb), nb)
    torch.cuda.synchronize()
    acc, bon = acc.cpu().numpy(), bon.cpu().numpy()
    first = np.where(acc >= 1, draft[:, 0], bon)
    p = softmax(T0[0].astype(np.float64) / temp)
    obs = np.bincount(first, minlength=V).astype(np.float64)
    exp = p * B
    big = exp >= 5
    stat = (((obs[big] - exp[big]) ** 2) / exp[big]).sum()
    rest_o, rest_e = obs[~big].sum(), exp[~big].sum()
    if rest_e > 0:
        stat += (rest_o - rest_e) ** 2 / rest_e
    dof = int(big.sum()) + (1 if rest_e > 0 else 0) - 1
    pval = chi2.sf(stat, dof)
    say(f"  acceptance rate {np.mean(acc >= 1):.3f}, chi2 {stat:.1f} on {dof} dof, p-value {pval:.3g}")
    assert pval > 1e-4
    # and the proposal alone is far from the target (the check has power)
    qfull = np.zeros(V)
    qfull[ids] = qp
    assert 0.5 * np.abs(qfull - p).sum() > 0.2
