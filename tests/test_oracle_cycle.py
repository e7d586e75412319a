"""Pins of the oracle's drafting cycle (draft -> verify -> inject), CPU only.

advance() is checked against its definition on hand cases and at its clamps; the cycle
driver is checked on a tiny fp32 drafter with target logits planted so that a chosen
number of drafts is accepted each cycle: the accepted prefix, the emitted tokens (the
target's greedy tokens, so decoding stays lossless), the positions of the injected rows
and the hand-over of the bonus token as the next anchor all follow from the definitions.
"""
import numpy as np

import oracle
import synth


def test_advance_hand_cases():
    o = oracle.advance(3, 77, 10, 1023, 100)
    assert (o["pos0"], o["n_new"], o["ctx_len"]) == (10, 4, 14)
    assert o["block_ids"].tolist() == [77] + [1023] * 15
    assert oracle.advance(0, 5, 0, 9, 64)["n_new"] == 1              # nothing accepted: the anchor row only
    assert oracle.advance(15, 5, 0, 9, 64)["ctx_len"] == 16          # every draft accepted


def test_advance_clamps():
    assert oracle.advance(-2, 1, 10, 9, 100)["n_new"] == 1
    assert oracle.advance(40, 1, 10, 9, 100)["n_new"] == 16
    o = oracle.advance(5, 1, 98, 9, 100)
    assert (o["pos0"], o["ctx_len"]) == (98, 100)                   # saturates at the capacity
    o = oracle.advance(2, 1, -5, 9, 100)
    assert (o["pos0"], o["ctx_len"]) == (0, 3)
    assert oracle.advance(2, 1, 500, 9, 100)["pos0"] == 100


def _planted(dims, accept_plan, seed):
    """Target logits accepting accept_plan[c] drafts in cycle c: row i < A carries a large
    logit on the draft token, row A on another token."""
    rng = np.random.default_rng(seed)
    bonus_tok = {}

    def logits_fn(c, path):
        A = accept_plan[c]
        T = rng.standard_normal((len(path) + 1, dims.vocab))
        for i in range(A):
            T[i, path[i]] = 50.0
        x = int((path[A] + 1 + c) % (dims.vocab - 1)) if A < len(path) else int(rng.integers(0, dims.vocab - 1))
        T[A, x] = 50.0
        bonus_tok[c] = x
        return T
    return logits_fn, bonus_tok


def test_cycle_planted_acceptance():
    wl = synth.workload("c1")
    dims = wl.dims
    W = synth.make_weights(dims, 5, ps_scale="stress")
    m = oracle.Model(dims, W)
    cap, L = 160, 40
    K, V = synth.make_cache(dims, [L], cap, 6, std=0.5)
    kc = [oracle.decode(K[l, 0], dims.dtype).copy() for l in range(dims.n_layers)]
    vc = [oracle.decode(V[l, 0], dims.dtype).copy() for l in range(dims.n_layers)]
    hidden = synth.make_hidden(dims, 16 * 4, 7)
    plan = [3, 0, 15, 7]
    logits_fn, bonus_tok = _planted(dims, plan, 8)
    ids0 = synth.make_block_ids(dims, 1, 9, 1)[0]
    out = oracle.drafting_cycles(m, kc, vc, L, cap, L - 16, 16, ids0,
                                 lambda c, n: hidden[16 * c:16 * c + n],
                                 logits_fn, len(plan))
    ctx = L
    for c, o in enumerate(out):
        A = plan[c]
        assert o["accept_len"] == A
        assert o["bonus"] == bonus_tok[c]
        assert o["emitted"] == list(o["path_ids"][:A]) + [bonus_tok[c]]
        # lossless: every emitted token is the target's greedy token of its row
        T = o["target_logits"]
        assert all(int(np.argmax(T[i])) == tok for i, tok in enumerate(o["emitted"]))
        assert o["ctx_len"] == ctx
        nxt = o["next"]
        assert (nxt["pos0"], nxt["n_new"], nxt["ctx_len"]) == (ctx, A + 1, ctx + A + 1)
        assert nxt["block_ids"][0] == o["bonus"]
        if c + 1 < len(out):
            assert out[c + 1]["pos0"] == ctx and out[c + 1]["n_new"] == A + 1
        ctx += A + 1
    # the rows injected by the last cycles sit right after the original context
    assert ctx == L + sum(a + 1 for a in plan)
