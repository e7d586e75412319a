"""Pins of the oracle's stated readings of the layer internals (CPU only).

The pages name the parts of a drafter layer (GQA attention over the injected context,
a SwiGLU feed-forward block, rotary positions, the Path Selector's context gate, the
two-tap short conv) without printing their numbers.  The oracle fixes one reading of
each; these tests tie that reading to closed forms built from library routines
(``torch.nn.functional.silu``, ``torch.sigmoid``, ``math.cos``/``math.sin``) on
single-coordinate weights, so that a slip in the oracle -- gate and up swapped, block
rows placed at positions ``j`` instead of ``ctx_len + j``, the gate's sigmoid negated
or read from the left neighbour, the conv's two correction halves swapped, the
injected keys rotated by the wrong angle -- fails one of them.

They also pin the small float32 helpers the GPU tests use to check a device result
against its own inputs (``tests/helpers.py``: ``walk_f32``, ``accept_of``,
``draw_f32``) to the oracle's ``select_path``, ``verify`` and sampling rule, on inputs
where float32 arithmetic is exact.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.dflash_ref import _inverse_cdf
from tests import helpers as H


def dims_of(**kw):
    base = dict(dtype="bf16", d=64, n_heads=4, n_kv_heads=2, head_dim=16, d_ffn=96, n_layers=1,
                n_feat_layers=2, d_target=32, vocab=200, ps_rank=4)
    base.update(kw)
    return synth.Dims(**base)


def put(w, name, idx, value, dtype="bf16"):
    """Set one element of a stored weight (bf16 bits) to ``value`` (a bf16-exact number)."""
    a = w[name]
    if dtype == "bf16":
        a[idx] = synth.f32_to_bf16_bits(np.array([value], dtype=np.float32))[0]
    else:
        a[idx] = np.float32(value)


def bf(x):
    """Library bf16 rounding (torch's float -> bfloat16 cast), back to float64."""
    return torch.tensor(np.asarray(x, dtype=np.float64)).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


def rot(v, ang):
    """A 2-vector turned by ``ang`` radians."""
    c, s = math.cos(ang), math.sin(ang)
    return np.array([c * v[0] - s * v[1], s * v[0] + c * v[1]])


# ------------------------------------------------------------------ SwiGLU: which projection is gated

def test_swiglu_gate_and_up_roles_against_library_silu():
    dims = dims_of(n_layers=1)
    everything = list(synth.weight_shapes(dims))
    zero = [n for n in everything if n.split(".")[-1] in ("w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down")]
    w = synth.make_weights(dims, 31, zero=zero)
    i, a, b, c = 70, 3, 11, 5          # hidden unit i >= d, so a transposed w_down would not reach column c
    put(w, "l0.w_gate", (i, a), 1.5)
    put(w, "l0.w_up", (i, b), -0.75)
    put(w, "l0.w_down", (c, i), 2.0)
    m = oracle.Model(dims, w)
    K, V = synth.make_cache(dims, [5], 32, 32)
    ids = synth.make_block_ids(dims, 1, 33)[0]
    ids[1:] = np.arange(1, 16) * 7      # distinct rows so every row has its own u
    out = oracle.draft_block(m, [oracle.decode(K[0, 0], "bf16")], [oracle.decode(V[0, 0], "bf16")], 5, ids)
    f = out["stream"][1] - out["stream"][0]          # attention sublayer is silent (w_o = 0)
    x = m.rows("embed", ids)
    u = bf(x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + dims.rms_eps))   # g_ffn = 1
    gate = torch.nn.functional.silu(torch.tensor(1.5 * u[:, a])).numpy()
    want_c = 2.0 * bf(gate * (-0.75 * u[:, b]))
    want = np.zeros_like(f)
    want[:, c] = want_c
    np.testing.assert_allclose(f, want, rtol=1e-12, atol=1e-12)
    # the swapped reading (SiLU on the up projection) gives other numbers on these inputs
    swapped = 2.0 * bf(torch.nn.functional.silu(torch.tensor(-0.75 * u[:, b])).numpy() * (1.5 * u[:, a]))
    assert np.abs(swapped - want_c).max() > 1e-2 * np.abs(want_c).max()


# ------------------------------------------------------------------ positions of the block rows

def _rope_dims():
    # one query head, one kv head of width 2: a single rotary pair turning at 1 rad per position
    return dims_of(d=8, n_heads=1, n_kv_heads=1, head_dim=2, d_ffn=8, vocab=64, ps_rank=2)


def _rope_weights(dims, seed, with_block_keys):
    names = list(synth.weight_shapes(dims))
    zero = [n for n in names if n.split(".")[-1] in ("w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down", "embed")]
    w = synth.make_weights(dims, seed, zero=zero)
    tok = 9
    put(w, "embed", (tok, 0), 1.0)
    put(w, "embed", (tok, 1), 0.5)     # E[tok] = (1, 0.5, 0, ...): u = rmsnorm of it
    put(w, "l0.w_q", (0, 0), 2.0)
    put(w, "l0.w_q", (1, 1), -3.0)
    if with_block_keys:
        put(w, "l0.w_k", (0, 1), 0.25)
        put(w, "l0.w_k", (1, 0), 0.125)
        put(w, "l0.w_v", (0, 0), 1.0)
    put(w, "l0.w_o", (0, 0), 1.0)
    put(w, "l0.w_o", (1, 1), 1.0)
    return w, tok


def _u_of_token(dims):
    e = np.array([1.0, 0.5] + [0.0] * (dims.d - 2))
    return bf(e / math.sqrt(np.mean(e * e) + dims.rms_eps))       # g_attn = 1


def test_block_queries_sit_at_context_length_plus_row():
    """Score of block row j against a context key stored at position p depends on ctx_len + j - p."""
    dims = _rope_dims()
    w, tok = _rope_weights(dims, 34, with_block_keys=False)
    m = oracle.Model(dims, w)
    L, p = 53, 20
    kc = np.zeros((1, 64, 2))
    vc = np.zeros((1, 64, 2))
    kc[0, p] = bf(rot(np.array([0.75, -1.25]), p * 1.0))     # the stored key: post-RoPE at its own position
    vc[0, p] = [1.0, 0.0]
    ids = np.full(16, tok, dtype=np.int32)
    out = oracle.draft_block(m, [kc], [vc], L, ids)
    o = (out["stream"][1] - out["stream"][0])[:, :2]
    u = _u_of_token(dims)
    q0 = np.array([2.0 * u[0], -3.0 * u[1]])

    def expect(offset):
        want = np.zeros((16, 2))
        for j in range(16):
            q = bf(rot(q0, (offset + j) * 1.0))                  # the query turned to its position
            s = float(q @ kc[0, p]) / math.sqrt(2.0)
            # every other context row and every block row has a zero key (score 0) and zero value
            want[j, 0] = bf(math.exp(s) / (math.exp(s) + (L - 1) + 16))
        return want

    want = expect(L)
    np.testing.assert_allclose(o, want, rtol=2 ** -7, atol=1e-7)
    # placing the block at positions 0..15 (the other reading) moves these numbers
    assert np.abs(expect(0) - want).max() > 0.05


def test_block_keys_rotate_with_their_own_rows():
    """Block keys turn at ctx_len + j too, so block-to-block scores depend on j - i only."""
    dims = _rope_dims()
    w, tok = _rope_weights(dims, 35, with_block_keys=True)
    m = oracle.Model(dims, w)
    ids = np.full(16, tok, dtype=np.int32)
    u = _u_of_token(dims)
    q0 = np.array([2.0 * u[0], -3.0 * u[1]])
    k0 = np.array([0.25 * u[1], 0.125 * u[0]])
    v0 = bf(u[0])

    def expect(L, key_offset):
        want = np.empty(16)
        for i in range(16):
            q = bf(rot(q0, (L + i) * 1.0))
            s = np.array([float(q @ bf(rot(k0, (key_offset + j) * 1.0))) / math.sqrt(2.0) for j in range(16)])
            want[i] = bf(v0 * np.exp(s).sum() / (np.exp(s).sum() + L))
        return want

    for L in (0, 37, 1001):
        kc = np.zeros((1, 1040, 2))      # context keys and values zero: score 0, no value
        vc = np.zeros((1, 1040, 2))
        out = oracle.draft_block(m, [kc], [vc], L, ids)
        o = (out["stream"][1] - out["stream"][0])[:, 0]
        want = expect(L, L)
        np.testing.assert_allclose(o, want, rtol=2 ** -7, atol=1e-7)
        if L:
            # keys at positions j with queries at ctx_len + i: a different result
            assert np.abs(expect(L, 0) - want).max() > 2 ** -4 * np.abs(want).max()


def test_injected_keys_turn_by_their_cache_position():
    """A key injected at position p, dotted with a query rotated to p + delta, equals the
    unrotated dot product turned by delta only (RoPE's relative property, with the query's
    rotation taken from the separately pinned ``oracle.rope``)."""
    dims = dims_of(d=32, d_target=32, n_heads=2, n_kv_heads=1, head_dim=16)
    w = synth.make_weights(dims, 36)
    eye = np.zeros((dims.d, dims.d_cat), dtype=np.float32)
    eye[:, :dims.d] = np.eye(dims.d, dtype=np.float32)
    w["w_fc"] = synth.f32_to_bf16_bits(eye)
    m = oracle.Model(dims, w)
    hid = synth.make_hidden(dims, 3, 37)
    pos = np.array([7, 4096, 12345])
    F, K, _ = oracle.inject_rows(m, hid, pos)
    k_plain = (F @ m.w("l0.w_k").T).reshape(3, 1, 16)          # before rotation
    r = np.random.default_rng(38)
    misses = []
    for i, p in enumerate(pos):
        for delta in (0, 5):
            q = r.standard_normal((1, 1, 16))
            got = float((oracle.rope(q, np.array([p + delta]), dims.rope_theta) * K[0, i]).sum())
            want = float((oracle.rope(q, np.array([delta]), dims.rope_theta) * k_plain[i]).sum())
            scale = np.linalg.norm(q) * np.linalg.norm(k_plain[i])
            assert abs(got - want) <= 2 ** -7 * scale, (p, delta, got, want)
            misses.append(abs(float((oracle.rope(q, np.array([p + delta]), dims.rope_theta) * k_plain[i]).sum())
                              - want) / scale)
    # a key left unrotated misses the relative property by far more than rounding
    assert max(misses) > 2 ** -3


# ------------------------------------------------------------------ the Path Selector's context gate

def _gate_model(seed=40):
    dims = dims_of(use_gate=True, ps_rank=1)
    names = list(synth.weight_shapes(dims))
    zero = [n for n in names if n in ("ps_left", "ps_right", "ps_u", "ps_v", "ps_gate")]
    w = synth.make_weights(dims, seed, zero=zero)
    k, cl, cr, cg = 7, 2, 9, 4
    put(w, "ps_left", (k, cl), 1.0)
    put(w, "ps_right", (k, cr), 1.0)
    put(w, "ps_u", (0, k), 1.0)
    put(w, "ps_v", (0, k), 1.0)
    put(w, "ps_gate", (k, cg), 3.0)
    return dims, oracle.Model(dims, w), (k, cl, cr, cg)


def test_gate_is_sigmoid_of_the_right_rows_hidden_state():
    dims, m, (k, cl, cr, cg) = _gate_model()
    ids, _, xh = synth.make_candidates(dims, 1, 41)
    bids = np.full(16, 5, dtype=np.int32)
    bids[0] = 17
    S = oracle.path_pair_scores(m, ids[0], xh[0], bids, 1)
    E = m.w("embed")
    gamma = torch.sigmoid(torch.tensor(3.0 * bf(xh[0, 1:, cg]))).numpy()      # drafted rows 1..15
    want = np.zeros_like(S)
    want[0, 0] = E[bids[0], cl] * E[ids[0, 1], cr] * gamma[0]
    for p in range(1, 15):
        want[p] = np.outer(E[ids[0, p], cl], E[ids[0, p + 1], cr] * gamma[p])
    np.testing.assert_allclose(S, want, rtol=1e-12, atol=1e-15)
    # sigma(-z) = 1 - sigma(z) would give other scores
    assert np.abs(1 - gamma - gamma).max() > 0.1


def test_gate_reads_only_its_own_position():
    dims, m, (k, cl, cr, cg) = _gate_model()
    ids, _, xh = synth.make_candidates(dims, 1, 42)
    bids = np.full(16, 5, dtype=np.int32)
    S = oracle.path_pair_scores(m, ids[0], xh[0], bids, 1)
    for row in (3, 9):                    # block row r = drafted position r - 1
        x2 = xh[0].copy()
        x2[row, cg] += 2.0
        S2 = oracle.path_pair_scores(m, ids[0], x2, bids, 1)
        changed = np.flatnonzero(np.abs(S2 - S).reshape(15, -1).max(axis=1) > 0)
        assert changed.tolist() == [row - 1], (row, changed)


# ------------------------------------------------------------------ the short conv's two correction halves

def _conv_dims():
    return dims_of(d=64, use_conv=True)


@pytest.mark.parametrize("live_half", ["a", "b"])
def test_conv_first_half_scales_current_row_second_half_previous(live_half):
    dims = _conv_dims()
    d, ng = dims.d, dims.d // 16
    w = synth.make_weights(dims, 43, zero=["l0.conv0.w0", "l0.conv0.w1", "l0.conv0.gen"])
    r = np.random.default_rng(44)
    gen = np.zeros((2 * ng, d), dtype=np.float32)
    rows = slice(0, ng) if live_half == "a" else slice(ng, 2 * ng)
    gen[rows] = (r.standard_normal((ng, d)) * 0.1).astype(np.float32)
    w["l0.conv0.gen"] = synth.f32_to_bf16_bits(gen)
    m = oracle.Model(dims, w)
    gq = m.w("l0.conv0.gen")
    u = np.zeros((16, d))
    u[0] = r.uniform(0.5, 1.5, d)
    u[1] = r.uniform(-1.5, -0.5, d)
    y = oracle.short_conv(m, 0, 0, u)
    delta1 = bf(u[1]) @ gq.T                                   # the correction of row 1, from row 1 itself
    grp = np.arange(d) // 16
    if live_half == "a":       # first half: tap on the current row
        want = u[1] + delta1[grp] * u[1]
        wrong = u[1] + delta1[grp] * u[0]
    else:                      # second half: tap on the previous row
        want = u[1] + delta1[ng + grp] * u[0]
        wrong = u[1] + delta1[ng + grp] * u[1]
    np.testing.assert_allclose(y[1], want, rtol=1e-13)
    assert np.abs(wrong - want).max() > 1e-3
    # a correction computed from the previous row instead would differ too
    delta0 = bf(u[0]) @ gq.T
    assert np.abs(delta0 - delta1).max() > 1e-3


# ------------------------------------------------------------------ the GPU tests' float32 helpers

def test_walk_f32_equals_oracle_select_path_on_exact_inputs():
    r = np.random.default_rng(45)
    for trial in range(60):
        P = int(r.integers(1, 16))
        lg = np.sort(r.integers(-8, 9, size=(P, 16)) / 4.0, axis=1)[:, ::-1].copy()   # quarters: exact sums
        S = r.integers(-6, 7, size=(P, 16, 16)) / 4.0
        anchor = bool(trial % 2)
        if not anchor:
            S[0] = 0.0
        for mode in ("greedy", "exact"):
            want, _ = oracle.select_path(lg, S, anchor, mode)
            np.testing.assert_array_equal(H.walk_f32(lg, S, anchor, mode), want, err_msg=f"{trial} {mode}")


def test_accept_of_equals_oracle_verify_with_ties():
    r = np.random.default_rng(46)
    for trial in range(80):
        P = int(r.integers(0, 16))
        T = r.integers(-3, 4, size=(P + 1, 40)).astype(np.float64)     # many exact ties
        greedy = [int(np.flatnonzero(row == row.max())[0]) for row in T]
        A = int(r.integers(0, P + 1))
        draft = np.array([greedy[i] if i < A else (greedy[i] + 1 + int(r.integers(0, 38))) % 40 for i in range(P)],
                         dtype=np.int32)
        assert H.accept_of(draft, T) == oracle.verify(draft, T)


def test_draw_f32_equals_oracle_inverse_cdf_on_exact_inputs():
    r = np.random.default_rng(47)
    for trial in range(200):
        q = r.integers(0, 5, size=16).astype(np.float64)
        if q.sum() == 0:
            q[3] = 1
        q = q / 64.0                                     # sixty-fourths: every partial sum exact
        u = float(r.integers(0, 64)) / 64.0              # lands on boundaries too
        assert H.draw_f32(q, u) == _inverse_cdf(q, u), (q, u)
    # the sampled walk draws with that rule from its own softmax
    dims = dims_of()
    lg = np.sort(r.standard_normal((6, 16)), axis=1)[:, ::-1].copy()
    S = r.standard_normal((6, 16, 16))
    uni = r.uniform(0.05, 0.95, 6)
    idx, q = oracle.sample_path(lg, S, True, 0.7, uni)
    for p in range(6):
        assert H.draw_f32(q[p], uni[p]) == idx[p]
