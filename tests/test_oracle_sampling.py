"""Pins of the oracle's sampled path choice and rejection-sampling verification.

The checks do not retype the oracle's formulas: they run the oracle over a fine grid of
its uniform inputs and compare the resulting frequencies with distributions computed by
a library routine (``scipy.special.softmax``), and check limits that reduce to the
greedy rules (pinned elsewhere).  The central one is the property that defines rejection
sampling: whatever the proposal, the first emitted token is distributed exactly as the
target's own distribution.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle

N = 2000
GRID = (np.arange(N) + 0.5) / N          # midpoints: a frequency is exact to 1/N


def _scores(seed, P=5, K=16):
    r = np.random.default_rng(seed)
    lg = np.sort(r.normal(0, 2, size=(P, K)))[:, ::-1].copy()
    S = r.normal(0, 1, size=(P, K, K))
    return lg, S


@pytest.mark.parametrize("anchor", [True, False])
def test_sample_path_cold_limit_is_greedy(anchor):
    for seed in range(5):
        lg, S = _scores(seed)
        u = np.random.default_rng(100 + seed).uniform(size=len(lg))
        idx, q = oracle.sample_path(lg, S, anchor, 1e-7, u)
        g, _ = oracle.select_path(lg, S, anchor, "greedy")
        np.testing.assert_array_equal(idx, g)
        np.testing.assert_allclose(q.sum(axis=1), 1.0, atol=1e-12)


@pytest.mark.parametrize("t", [0.5, 1.0, 3.0])
def test_sample_path_draw_frequencies(t):
    lg, S = _scores(7, P=3)
    # position 0 (anchor row of the pair scores): frequencies over the grid
    hits = np.zeros(16)
    for u0 in GRID:
        idx, _ = oracle.sample_path(lg, S, True, t, np.array([u0, 0.5, 0.5]))
        hits[idx[0]] += 1
    want0 = softmax((lg[0] + S[0, 0]) / t)
    np.testing.assert_allclose(hits / N, want0, atol=1.5 / N)
    # position 1 given the draw at 0: the scores pair the drawn left candidate (row of S[1])
    u0 = 0.3
    prev = oracle.sample_path(lg, S, True, t, np.array([u0, 0.5, 0.5]))[0][0]
    hits = np.zeros(16)
    q1 = None
    for u1 in GRID:
        idx, q = oracle.sample_path(lg, S, True, t, np.array([u0, u1, 0.5]))
        hits[idx[1]] += 1
        q1 = q[1]
    want1 = softmax((lg[1] + S[1, prev]) / t)
    np.testing.assert_allclose(hits / N, want1, atol=1.5 / N)
    np.testing.assert_allclose(q1, want1, rtol=1e-10, atol=1e-15)
    # without an anchor position 0 has no pair term
    idx, q = oracle.sample_path(lg, S, False, t, np.array([0.5, 0.5, 0.5]))
    np.testing.assert_allclose(q[0], softmax(lg[0] / t), rtol=1e-10, atol=1e-15)


def _verify_case(seed, V=10, P=3, K=4, t=1.0):
    """Target logits, sparse proposals that over-weight some tokens (so rejections happen),
    and drafts drawn from the proposals."""
    r = np.random.default_rng(seed)
    T = r.normal(0, 1.5, size=(P + 1, V))
    q_ids = np.stack([r.permutation(V)[:K] for _ in range(P)]).astype(np.int32)
    q_probs = r.dirichlet(np.full(K, 0.5), size=P)
    draft = np.array([q_ids[i][np.argmax(q_probs[i])] for i in range(P)], dtype=np.int32)
    return T, q_ids, q_probs, draft, t


def _emitted_given_draft(T, q_ids, q_probs, draft, t, pos):
    """Distribution of the emitted token at block position ``pos`` for a fixed draft,
    given that every draft before it was accepted, from the oracle's decisions over grids
    of its uniforms; and the acceptance frequency of draft[pos]."""
    P = len(draft)
    base = np.zeros(P)                     # u = 0 accepts any draft with p > 0 and q > 0
    acc = []
    for u in GRID:
        ua = base.copy()
        ua[pos] = u
        a, _ = oracle.verify_sampled(draft, q_ids, q_probs, T, t, ua, 0.5)
        assert a >= pos
        acc.append(a > pos)
    acc = np.asarray(acc)
    out = np.zeros(T.shape[1])
    out[draft[pos]] += acc.mean()
    if (~acc).any():
        ua = base.copy()
        ua[pos] = GRID[np.flatnonzero(~acc)[0]]
        hist = np.zeros(T.shape[1])
        for ub in GRID:
            a, bonus = oracle.verify_sampled(draft, q_ids, q_probs, T, t, ua, ub)
            assert a == pos
            hist[bonus] += 1
        out += (~acc).mean() * hist / N
    return out, acc.mean()


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("t", [0.7, 1.0])
def test_verify_sampled_is_lossless(seed, t):
    """With the draft token drawn from its proposal, the emitted token at each position is
    distributed as the target's softmax, whatever the proposal."""
    T, q_ids, q_probs, draft, t = _verify_case(seed, t=t)
    rejected_somewhere = False
    for pos in range(2):
        p = softmax(T[pos] / t)
        mix = np.zeros(T.shape[1])
        for j, x in enumerate(q_ids[pos]):
            d = draft.copy()
            d[pos] = x
            got, acc = _emitted_given_draft(T, q_ids, q_probs, d, t, pos)
            # the draft is accepted with probability min(1, p/q)
            assert abs(acc - min(1.0, p[x] / q_probs[pos][j])) <= 1.0 / N
            rejected_somewhere |= acc < 1.0
            mix += q_probs[pos][j] * got
        np.testing.assert_allclose(mix, p, atol=3.0 / N)
    assert rejected_somewhere               # the case exercises the residual draw


def test_verify_sampled_exact_proposal_accepts_everything():
    r = np.random.default_rng(5)
    V, P, t = 8, 4, 1.0
    T = r.normal(0, 1, size=(P + 1, V))
    q_ids = np.tile(np.arange(V, dtype=np.int32), (P, 1))
    q_probs = np.stack([softmax(T[i] / t) for i in range(P)])
    draft = np.array([r.integers(V) for _ in range(P)], dtype=np.int32)
    hist = np.zeros(V)
    for k, u in enumerate(GRID):
        a, bonus = oracle.verify_sampled(draft, q_ids, q_probs, T, t, np.full(P, GRID[(7 * k) % N]), u)
        assert a == P
        hist[bonus] += 1
    np.testing.assert_allclose(hist / N, softmax(T[P] / t), atol=1.5 / N)


def test_verify_sampled_cold_limit_is_greedy():
    r = np.random.default_rng(11)
    V, P, K = 50, 6, 8
    for case in range(20):
        T = r.normal(0, 1, size=(P + 1, V))
        greedy = T.argmax(axis=1)
        n_ok = r.integers(0, P + 1)
        draft = np.array([greedy[i] if i < n_ok else (greedy[i] + 1 + r.integers(V - 1)) % V for i in range(P)],
                         dtype=np.int32)
        q_ids = np.zeros((P, K), dtype=np.int32)
        for i in range(P):
            others = r.permutation([v for v in range(V) if v != draft[i]])[:K - 1]
            q_ids[i] = np.concatenate([[draft[i]], others])[r.permutation(K)]
        q_probs = r.dirichlet(np.ones(K), size=P)
        got = oracle.verify_sampled(draft, q_ids, q_probs, T, 1e-5, r.uniform(size=P), r.uniform())
        assert got == oracle.verify(draft, T), case


def test_verify_sampled_edges():
    r = np.random.default_rng(3)
    V, t = 6, 1.0
    T = r.normal(0, 1, size=(3, V))
    q_ids = np.array([[0, 1], [2, 3]], dtype=np.int32)
    q_probs = np.array([[0.5, 0.5], [0.5, 0.5]])
    # a draft token the proposal never lists is rejected, whatever the uniform
    a, _ = oracle.verify_sampled(np.array([4, 2]), q_ids, q_probs, T, t, np.zeros(2), 0.5)
    assert a == 0
    # no drafts: the bonus is a draw from row 0
    hist = np.zeros(V)
    for u in GRID:
        a, b = oracle.verify_sampled(np.zeros(0, dtype=np.int32), q_ids[:0], q_probs[:0], T[:1], t,
                                     np.zeros(0), u)
        assert a == 0
        hist[b] += 1
    np.testing.assert_allclose(hist / N, softmax(T[0] / t), atol=1.5 / N)
    with pytest.raises(ValueError):
        oracle.verify_sampled(np.array([0]), q_ids[:1], q_probs[:1], T[:2], 0.0, np.zeros(1), 0.5)
    with pytest.raises(ValueError):
        oracle.sample_path(np.zeros((2, 16)), np.zeros((2, 16, 16)), True, -1.0, np.zeros(2))
