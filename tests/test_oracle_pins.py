"""Pins of the CPU oracle to facts other than itself (CPU only).

Each test checks the oracle against something the pages or the mathematics fix:
closed forms, special cases that reduce to a library routine, brute force on tiny
inputs, invariants, hand-worked examples from ``tests/golden`` and the parameter
counts printed in the DFlash 2 article's layer/technology table.  Each is chosen so
that a plausible slip in the oracle (a dropped term, a wrong sign, index or
operand order) fails at least one of them.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny_dims(**kw):
    base = dict(dtype="bf16", d=64, n_heads=4, n_kv_heads=2, head_dim=16, d_ffn=96, n_layers=1,
                n_feat_layers=2, d_target=32, vocab=200, ps_rank=4)
    base.update(kw)
    return synth.Dims(**base)


def rng(seed=0):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------ number formats

def test_bf16_round_hand_values():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -7, -(1 + 2 ** -8) - 2 ** -20, 0.0, 2.0 ** 130])
    want = np.array([1.0, 1.0, 1 + 2 ** -6, 1 + 2 ** -7, -(1 + 2 ** -7), 0.0, np.inf])
    np.testing.assert_array_equal(oracle.bf16_round(x), want)


def test_bf16_round_matches_library_conversion():
    # torch's float32 -> bfloat16 cast rounds to nearest even: a library routine.
    v = rng(1).standard_normal(200000).astype(np.float32) * np.float32(37.0)
    v[:1000] = rng(2).standard_normal(1000).astype(np.float32) * np.float32(1e-39)   # subnormals
    lib = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.bf16_round(v.astype(np.float64)), lib)


def test_decode_bits():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x4049], dtype=np.uint16)
    np.testing.assert_array_equal(oracle.decode(bits, "bf16"), [1.0, -2.0, 0.0, 3.140625])


# ------------------------------------------------------------------ rmsnorm, rope

def test_rmsnorm_hand_example_and_invariance():
    v = np.array([[3.0, 4.0]])
    np.testing.assert_allclose(oracle.rmsnorm(v, np.array([1.0, 2.0]), 0.0),
                               [[3 / math.sqrt(12.5), 8 / math.sqrt(12.5)]], rtol=1e-15)
    x = rng(3).standard_normal((5, 64))
    g = rng(4).standard_normal(64)
    np.testing.assert_allclose(oracle.rmsnorm(7.5 * x, g, 0.0), oracle.rmsnorm(x, g, 0.0), rtol=1e-13)
    c = 0.3
    np.testing.assert_allclose(oracle.rmsnorm(np.full((1, 8), c), np.ones(8), 1e-6), c / math.sqrt(c * c + 1e-6))


def test_rope_closed_forms():
    # one pair, inverse frequency 1: a plain 2-d rotation by `pos` radians
    x = np.array([[[1.0, 0.0]]])
    for p in (0.0, 1.0, 2.5):
        np.testing.assert_allclose(oracle.rope(x, np.array([p]), 1e6)[0, 0], [math.cos(p), math.sin(p)], atol=1e-15)
    # rotate-half pairing: dim 0 pairs with dim hd/2 (not dim 1)
    x = np.array([[[1.0, 0.0, 0.0, 0.0]]])
    p = 0.7
    np.testing.assert_allclose(oracle.rope(x, np.array([p]), 1e6)[0, 0], [math.cos(p), 0, math.sin(p), 0], atol=1e-15)
    # second pair turns at theta^(-2/hd)
    x = np.array([[[0.0, 1.0, 0.0, 0.0]]])
    f = 100.0 ** (-0.5)
    np.testing.assert_allclose(oracle.rope(x, np.array([3.0]), 100.0)[0, 0],
                               [0, math.cos(3 * f), 0, math.sin(3 * f)], atol=1e-15)


def test_rope_relative_and_norm():
    r = rng(5)
    q = r.standard_normal((1, 1, 32))
    k = r.standard_normal((1, 1, 32))
    dots = []
    for shift in (0, 17, 4000):
        qq = oracle.rope(q, np.array([10 + shift]), 1e6)
        kk = oracle.rope(k, np.array([3 + shift]), 1e6)
        dots.append(float((qq * kk).sum()))
        np.testing.assert_allclose(np.linalg.norm(qq), np.linalg.norm(q), rtol=1e-13)
    np.testing.assert_allclose(dots, dots[0], rtol=1e-10)
    np.testing.assert_array_equal(oracle.rope(q, np.array([0]), 1e6), q)


# ------------------------------------------------------------------ fusion + injection

def _model(dims, seed=0, **kw):
    return oracle.Model(dims, synth.make_weights(dims, seed, **kw))


def test_inject_identity_fusion_special_case():
    dims = tiny_dims(d=32, d_target=32)
    w = synth.make_weights(dims, 1)
    eye = np.zeros((dims.d, dims.d_cat), dtype=np.float32)
    eye[:, :dims.d] = np.eye(dims.d, dtype=np.float32)
    w["w_fc"] = synth.f32_to_bf16_bits(eye)
    m = oracle.Model(dims, w)
    hid = synth.make_hidden(dims, 5, 2)
    F, K, V = oracle.inject_rows(m, hid, np.arange(5))
    H = oracle.decode(hid, "bf16")[:, :dims.d]
    np.testing.assert_array_equal(F, oracle.bf16_round(oracle.rmsnorm(H, 1.0, dims.rms_eps)))
    # position 0 is not rotated: K equals the plain key projection there
    k0 = (F[:1] @ m.w("l0.w_k").T).reshape(1, dims.n_kv_heads, dims.head_dim)
    np.testing.assert_array_equal(K[0, :1], oracle.bf16_round(k0))
    np.testing.assert_array_equal(V[0], oracle.bf16_round((F @ m.w("l0.w_v").T).reshape(5, dims.n_kv_heads, dims.head_dim)))


def test_inject_row_independence_and_scale():
    dims = tiny_dims(n_layers=2)
    m = _model(dims, 3)
    hid = synth.make_hidden(dims, 9, 4)
    pos = np.arange(20, 29)
    F, K, V = oracle.inject_rows(m, hid, pos)
    F1, K1, V1 = oracle.inject_rows(m, hid[:4], pos[:4])
    F2, K2, V2 = oracle.inject_rows(m, hid[4:], pos[4:])
    np.testing.assert_allclose(np.concatenate([K1, K2], axis=1), K, rtol=1e-2, atol=1e-6)
    np.testing.assert_allclose(np.concatenate([V1, V2], axis=1), V, rtol=1e-2, atol=1e-6)
    # the fusion norm removes a positive scale of the hidden states (2x is exact in bf16)
    hid2 = synth.f32_to_bf16_bits(2 * synth.bits_to_f32(hid))
    Fs, _, _ = oracle.inject_rows(m, hid2, pos)
    np.testing.assert_allclose(Fs, F, rtol=1e-2)


# ------------------------------------------------------------------ dynamic short conv

def _conv_model(d=64, zero=(), seed=6):
    dims = tiny_dims(d=d, use_conv=True)
    return oracle.Model(dims, synth.make_weights(dims, seed, conv_scale="stress", zero=zero))


def test_conv_zero_taps_is_identity_exactly():
    zero = [f"l0.conv0.{k}" for k in ("gen", "w0", "w1")]
    m = _conv_model(zero=zero)
    u = rng(7).standard_normal((16, 64))
    np.testing.assert_array_equal(oracle.short_conv(m, 0, 0, u), u)


def test_conv_zero_generator_static_closed_form():
    m = _conv_model(zero=["l0.conv1.gen"])
    u = rng(8).standard_normal((16, 64))
    w0, w1 = m.w("l0.conv1.w0"), m.w("l0.conv1.w1")
    want = u + w0 * u
    want[1:] += w1 * u[:-1]
    np.testing.assert_allclose(oracle.short_conv(m, 0, 1, u), want, rtol=1e-14)


def test_conv_locality_and_group_sharing():
    m = _conv_model()
    d = 64
    u = np.zeros((16, d))
    u[5] = rng(9).standard_normal(d)
    y = oracle.short_conv(m, 0, 2, u)
    nz = np.flatnonzero(np.abs(y).sum(axis=1))
    assert set(nz) <= {5, 6}
    # the row after the impulse sees only the static previous-row tap (its own row is 0)
    np.testing.assert_allclose(y[6], m.w("l0.conv2.w1") * u[5], rtol=1e-14)
    # with zero static taps the correction on row 0 is one value per 16-channel group
    m0 = _conv_model(zero=["l0.conv3.w0", "l0.conv3.w1"])
    x = rng(10).uniform(0.5, 1.5, size=(16, d))
    y = oracle.short_conv(m0, 0, 3, x)
    ratio = (y[0] - x[0]) / x[0]
    grp = ratio.reshape(d // 16, 16)
    np.testing.assert_allclose(grp, grp[:, :1] * np.ones((1, 16)), rtol=1e-10, atol=1e-14)
    assert np.ptp(grp[:, 0]) > 1e-6


def test_conv_parameter_count_matches_page():
    # DFlash 2 article, layer/technology table: the dynamic short conv adds 16.5M parameters.
    # A 5-layer drafter of width 2560 with 4 conv sites per layer gives 16,486,400.
    assert oracle.conv_param_count(2560, 5) == 16_486_400
    assert round(oracle.conv_param_count(2560, 5) / 1e6, 1) == 16.5


# ------------------------------------------------------------------ block attention

def _rand_attn(seed, L, H=4, Hkv=2, hd=8, nq=16):
    r = rng(seed)
    return (r.standard_normal((nq, H, hd)), r.standard_normal((Hkv, L, hd)), r.standard_normal((Hkv, L, hd)),
            r.standard_normal((nq, Hkv, hd)), r.standard_normal((nq, Hkv, hd)))


def test_attention_empty_context_is_library_sdpa():
    q, kc, vc, kb, vb = _rand_attn(11, 0)
    got = oracle.block_attention(q, kc, vc, kb, vb)
    tq = torch.from_numpy(q).permute(1, 0, 2)                      # [H, 16, hd]
    tk = torch.from_numpy(kb).permute(1, 0, 2).repeat_interleave(2, dim=0)
    tv = torch.from_numpy(vb).permute(1, 0, 2).repeat_interleave(2, dim=0)
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=False)
    np.testing.assert_allclose(got, want.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_attention_identical_keys_average_values():
    q, kc, vc, kb, vb = _rand_attn(12, 10)
    kc[:] = 0.3
    kb[:] = 0.3
    got = oracle.block_attention(q, kc, vc, kb, vb)
    for h in range(4):
        g = h // 2
        mean = np.concatenate([vc[g], vb[:, g]]).mean(axis=0)
        np.testing.assert_allclose(got[:, h], np.broadcast_to(mean, (16, 8)), rtol=1e-12)


def test_attention_context_permutation_invariance():
    q, kc, vc, kb, vb = _rand_attn(13, 40)
    perm = rng(14).permutation(40)
    np.testing.assert_allclose(oracle.block_attention(q, kc[:, perm], vc[:, perm], kb, vb),
                               oracle.block_attention(q, kc, vc, kb, vb), rtol=1e-12)


def test_attention_bidirectional_in_block_and_full_context():
    q, kc, vc, kb, vb = _rand_attn(15, 30)
    base = oracle.block_attention(q, kc, vc, kb, vb)
    kb2 = kb.copy()
    kb2[12] += 1.0                                  # a later block row
    out = oracle.block_attention(q, kc, vc, kb2, vb)
    assert np.all(np.abs(out - base).max(axis=(1, 2))[:12] > 1e-6)   # earlier rows see it too
    vc2 = vc.copy()
    vc2[:, 29] += 1.0                               # the last context row
    out = oracle.block_attention(q, kc, vc2, kb, vb)
    assert np.all(np.abs(out - base).max(axis=(1, 2)) > 1e-6)


# ------------------------------------------------------------------ drafter forward

def test_draft_ignores_cache_rows_beyond_context():
    dims = tiny_dims(n_layers=2)
    m = _model(dims, 16)
    K, V = synth.make_cache(dims, [20], 64, 17)
    Kp, Vp = synth.make_cache(dims, [20], 64, 17, poison=True)
    ids = synth.make_block_ids(dims, 1, 18)[0]
    kc = [oracle.decode(K[l, 0], "bf16") for l in range(2)]
    vc = [oracle.decode(V[l, 0], "bf16") for l in range(2)]
    kp = [oracle.decode(Kp[l, 0], "bf16") for l in range(2)]
    vp = [oracle.decode(Vp[l, 0], "bf16") for l in range(2)]
    a = oracle.draft_block(m, kc, vc, 20, ids)["logits"]
    b = oracle.draft_block(m, kp, vp, 20, ids)["logits"]
    assert np.isfinite(b).all()
    np.testing.assert_array_equal(a, b)


def test_draft_with_silent_sublayers_is_embedding_head():
    dims = tiny_dims(n_layers=2)
    zero = [f"l{l}.{k}" for l in range(2) for k in ("w_o", "w_down")]
    m = _model(dims, 19, zero=zero)
    K, V = synth.make_cache(dims, [7], 32, 20)
    ids = synth.make_block_ids(dims, 1, 21)[0]
    out = oracle.draft_block(m, [oracle.decode(K[l, 0], "bf16") for l in range(2)],
                             [oracle.decode(V[l, 0], "bf16") for l in range(2)], 7, ids)
    x = m.rows("embed", ids)
    want = oracle.bf16_round(oracle.rmsnorm(x, 1.0, dims.rms_eps)) @ m.w("lm_head").T
    np.testing.assert_allclose(out["logits"], want, rtol=1e-12, atol=1e-12)


def test_draft_block_rows_see_later_rows():
    dims = tiny_dims()
    m = _model(dims, 22)
    K, V = synth.make_cache(dims, [9], 32, 23)
    kc = [oracle.decode(K[0, 0], "bf16")]
    vc = [oracle.decode(V[0, 0], "bf16")]
    ids = synth.make_block_ids(dims, 1, 24)[0]
    a = oracle.draft_block(m, kc, vc, 9, ids)["logits"]
    ids2 = ids.copy()
    ids2[15] = 3
    b = oracle.draft_block(m, kc, vc, 9, ids2)["logits"]
    assert np.abs(a[0] - b[0]).max() > 1e-9          # row 0 changes when row 15 changes


# ------------------------------------------------------------------ top-k

def test_topk_is_stable_full_sort():
    r = rng(25)
    lg = np.round(r.standard_normal((6, 500)) * 4) / 4          # many exact ties
    ids, vals = oracle.topk(lg, 16)
    for i in range(6):
        order = np.lexsort((np.arange(500), -lg[i]))[:16]
        np.testing.assert_array_equal(ids[i], order)
        np.testing.assert_array_equal(vals[i], lg[i, order].astype(np.float32))
        assert ids[i, 0] == int(np.argmax(lg[i]))


# ------------------------------------------------------------------ path selector

def test_path_selector_parameter_count_matches_page():
    # DFlash 2 article, layer/technology table: the Path Selector adds 2.0M parameters on
    # 256-d embeddings.  Width 2560, rank 64: 3*256*2560 + 2*64*256 = 1,998,848.
    assert oracle.path_selector_param_count(2560, 256, 64) == 1_998_848
    assert round(oracle.path_selector_param_count(2560, 256, 64) / 1e6, 1) == 2.0


def _ps_model(seed=26, **kw):
    dims = tiny_dims(**kw)
    return dims, oracle.Model(dims, synth.make_weights(dims, seed, ps_scale="stress"))


def test_pair_scores_are_rank_limited_and_role_symmetric():
    dims, m = _ps_model()
    ids, lg, xh = synth.make_candidates(dims, 1, 27)
    S = oracle.path_pair_scores(m, ids[0], xh[0], np.full(16, 5), 1)
    assert S.shape == (15, 16, 16)
    for p in range(1, 15):
        assert np.linalg.matrix_rank(S[p], tol=1e-9 * np.abs(S[p]).max()) <= dims.ps_rank
    assert np.abs(S[1:]).max() > 0.1
    # swapping the left/right roles transposes the ungated pair scores
    w2 = dict(m.stored)
    w2["ps_left"], w2["ps_right"] = m.stored["ps_right"], m.stored["ps_left"]
    w2["ps_u"], w2["ps_v"] = m.stored["ps_v"], m.stored["ps_u"]
    m2 = oracle.Model(dims, w2)
    c = ids[0].copy()
    c[2] = c[1]                 # block rows 1 and 2 = drafted positions 0 and 1
    S1 = oracle.path_pair_scores(m, c, xh[0], np.full(16, 5), 1)
    S2 = oracle.path_pair_scores(m2, c, xh[0], np.full(16, 5), 1)
    np.testing.assert_allclose(S2[1], S1[1].T, rtol=1e-10)
    assert np.abs(S1[1] - S1[1].T).max() > 1e-3


def test_gate_at_zero_halves_the_scores():
    dims, m = _ps_model()
    ids, _, xh = synth.make_candidates(dims, 1, 28)
    dg = tiny_dims(use_gate=True)
    w = dict(m.stored)
    w["ps_gate"] = synth.const(w["ps_gate"].shape, 0.0, "bf16")
    mg = oracle.Model(dg, w)
    S = oracle.path_pair_scores(m, ids[0], xh[0], np.full(16, 5), 1)
    Sg = oracle.path_pair_scores(mg, ids[0], xh[0], np.full(16, 5), 1)
    np.testing.assert_allclose(Sg, 0.5 * S, rtol=1e-12)


def test_zero_compatibility_picks_top_candidate():
    dims = tiny_dims()
    m = oracle.Model(dims, synth.make_weights(dims, 29, zero=["ps_u"]))
    ids, lg, xh = synth.make_candidates(dims, 1, 30)
    S = oracle.path_pair_scores(m, ids[0], xh[0], np.full(16, 5), 1)
    assert not S.any()
    for mode in ("greedy", "exact"):
        idx, _ = oracle.select_path(lg[0, 1:], S, True, mode)
        np.testing.assert_array_equal(idx, np.zeros(15))


def _brute(lg, S, anchor):
    P, K = lg.shape
    best, arg = -np.inf, None
    for path in itertools.product(range(K), repeat=P):
        s = lg[0, path[0]] + (S[0, 0, path[0]] if anchor else 0.0)
        for p in range(1, P):
            s += lg[p, path[p]] + S[p, path[p - 1], path[p]]
        if s > best:
            best, arg = s, path
    return np.asarray(arg), best


@pytest.mark.parametrize("K,P,anchor", [(4, 1, True), (4, 3, False), (4, 5, True), (3, 6, False), (16, 2, True), (16, 3, False)])
def test_exact_path_equals_brute_force(K, P, anchor):
    r = rng(K * 100 + P)
    for _ in range(5):
        lg = r.standard_normal((P, K))
        S = r.standard_normal((P, K, K)) * 1.5
        idx, tot = oracle.select_path(lg, S, anchor, "exact")
        bidx, btot = _brute(lg, S, anchor)
        np.testing.assert_allclose(tot, btot, rtol=1e-12)
        np.testing.assert_array_equal(idx, bidx)
        gidx, gtot = oracle.select_path(lg, S, anchor, "greedy")
        assert gtot <= btot + 1e-12
        # the greedy first pick is the best first-position score on its own
        first = lg[0] + (S[0, 0] if anchor else 0)
        assert gidx[0] == int(np.argmax(first))


def test_golden_greedy_vs_exact_counterexample():
    txt = open(os.path.join(GOLDEN, "path_counterexample.txt")).read().splitlines()
    kv = dict(l.split(" = ") for l in txt if " = " in l and not l.startswith("#"))
    lg = np.array([[float(v) for v in kv["logits0"].split()], [float(v) for v in kv["logits1"].split()]])
    S = np.zeros((2, 2, 2))
    S[1] = np.array([[float(v) for v in row.split()] for row in kv["S1"].split("/")])
    for mode in ("greedy", "exact"):
        path, total = kv[mode].split("/")
        idx, tot = oracle.select_path(lg, S, False, mode)
        np.testing.assert_array_equal(idx, [int(v) for v in path.split()])
        assert tot == float(total)


# ------------------------------------------------------------------ verification

def _golden_verify():
    for line in open(os.path.join(GOLDEN, "verify_cases.txt")):
        if line.startswith("#") or not line.strip():
            continue
        d, t, a, b = [f.split() for f in line.split("|")]
        yield [int(v) for v in d], [int(v) for v in t], int(a[0]), int(b[0])


def test_verify_golden_cases():
    for draft, tgt, a, bonus in _golden_verify():
        V = 12
        T = np.zeros((len(tgt), V))
        T[np.arange(len(tgt)), tgt] = 1.0
        assert oracle.verify(np.asarray(draft), T) == (a, bonus)


def test_verify_brute_force_and_invariants():
    r = rng(31)
    for trial in range(300):
        P = int(r.integers(0, 9))
        V = int(r.integers(2, 7))
        T = r.integers(0, 3, size=(P + 1, V)).astype(np.float64)     # frequent ties
        draft = r.integers(0, V, size=P)
        a, bonus = oracle.verify(draft, T)
        # brute force: the largest k whose prefix matches the lowest-index maxima
        greedy = [min(np.flatnonzero(T[i] == T[i].max())) for i in range(P + 1)]
        ks = [k for k in range(P + 1) if all(draft[i] == greedy[i] for i in range(k))]
        assert a == max(ks)
        assert bonus == greedy[a]
        assert 0 <= a <= P
        emitted = list(draft[:a]) + [bonus]
        assert emitted == greedy[:a + 1]                # lossless w.r.t. greedy target decoding
        T2 = T.copy()
        full = np.array(greedy[:P])
        assert oracle.verify(full, T2) == (P, greedy[P])


# ------------------------------------------------------------------ dynamic block size

@pytest.mark.parametrize("nq", [5, 8, 16])
def test_attention_any_block_size_is_library_sdpa(nq):
    """A block of nq rows attends to the whole context and its own nq rows: textbook
    attention over the concatenated keys (library routine, GQA by repeating kv heads)."""
    q, kc, vc, kb, vb = _rand_attn(40 + nq, 23, nq=nq)
    got = oracle.block_attention(q, kc, vc, kb, vb)
    assert got.shape == (nq, 4, 8)
    tq = torch.from_numpy(q).permute(1, 0, 2)                                   # [H, nq, hd]
    keys = np.concatenate([kc, kb.transpose(1, 0, 2)], axis=1)                 # [Hkv, L + nq, hd]
    vals = np.concatenate([vc, vb.transpose(1, 0, 2)], axis=1)
    tk = torch.from_numpy(keys).repeat_interleave(2, dim=0)
    tv = torch.from_numpy(vals).repeat_interleave(2, dim=0)
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=False)
    np.testing.assert_allclose(got, want.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("nb", [2, 5, 8])
def test_smaller_block_shapes_and_local_pair_scores(nb):
    """A block of nb < 16 rows drafts nb rows (positions L..L+nb-1), and its pair scores are
    those of the same positions in a 16-row block: each score reads only the candidates of
    its own and the previous position and the gate of its own row."""
    dims, m = _ps_model()
    ids, lg, xh = synth.make_candidates(dims, 1, 41)
    bids = np.full(16, dims.mask_id)
    bids[0] = 7
    S16 = oracle.path_pair_scores(m, ids[0], xh[0], bids, 1)
    Sn = oracle.path_pair_scores(m, ids[0][:nb], xh[0][:nb], bids[:nb], 1)
    assert Sn.shape == (nb - 1, 16, 16)
    np.testing.assert_allclose(Sn, S16[:nb - 1], rtol=1e-13, atol=1e-13)
    # the forward pass over nb rows: shapes, and the anchor row's positions start at L
    dims2 = tiny_dims(n_layers=1)
    m2 = oracle.Model(dims2, synth.make_weights(dims2, 3))
    K, V = synth.make_cache(dims2, [9], 64, 5)
    kc = [oracle.decode(K[0, 0], dims2.dtype)]
    vc = [oracle.decode(V[0, 0], dims2.dtype)]
    out = oracle.draft_block(m2, kc, vc, 9, bids[:nb])
    assert out["logits"].shape == (nb, dims2.vocab) and out["xhat"].shape == (nb, dims2.d)
    # attention inside the block is bidirectional at any size: a second row changes row 0
    one = oracle.draft_block(m2, kc, vc, 9, bids[:1])["logits"]
    two = oracle.draft_block(m2, kc, vc, 9, bids[:2])["logits"]
    assert np.abs(two[0] - one[0]).max() > 1e-9


# ------------------------------------------------------------------ bonus-guided calibration

def _cal_model(cal_dim=8, seed=50, **kw):
    dims = tiny_dims(**kw)
    W = synth.make_weights(dims, seed)
    W.update(synth.make_cal_weights(dims, seed, cal_dim, std=0.3))
    return dims, W


def test_calibration_zero_output_layer_is_identity():
    dims, W = _cal_model()
    W["cal_w2"] = synth.const(W["cal_w2"].shape, 0.0, dims.dtype)
    m = oracle.Model(dims, W)
    r = rng(51)
    xh, lg = r.standard_normal((16, dims.d)), r.standard_normal((16, dims.vocab))
    np.testing.assert_array_equal(oracle.calibrate(m, xh, 3, lg), lg)


def test_calibration_structure_against_library_silu():
    """W1 picking single input coordinates and W2 routing hidden unit k to token k: the
    bias of token k is silu of that coordinate (library silu).  Unit 0 reads the bonus
    embedding's first coordinate, unit 1 the row's own first hidden coordinate: this fixes
    the concatenation order [embedding; hidden]."""
    dims, W = _cal_model(cal_dim=4, dtype="f32")
    d = dims.d
    w1 = np.zeros((4, 2 * d), dtype=np.float32)
    w1[0, 0] = 1.0          # bonus embedding, coordinate 0
    w1[1, d] = 1.0          # hidden state, coordinate 0
    w1[2, d + 5] = -2.0     # hidden state, coordinate 5
    w2 = np.zeros((dims.vocab, 4), dtype=np.float32)
    w2[10, 0] = w2[11, 1] = w2[12, 2] = 1.0
    W["cal_w1"], W["cal_w2"] = w1, w2
    m = oracle.Model(dims, W)
    r = rng(52)
    xh = r.standard_normal((5, d))
    lg = np.zeros((5, dims.vocab))
    out = oracle.calibrate(m, xh, 7, lg)
    silu = torch.nn.functional.silu
    e = oracle.decode(W["embed"][7], "f32")
    np.testing.assert_allclose(out[:, 10], silu(torch.tensor(e[0])).item(), rtol=1e-12)
    np.testing.assert_allclose(out[:, 11], silu(torch.from_numpy(xh[:, 0])).numpy(), rtol=1e-12)
    np.testing.assert_allclose(out[:, 12], silu(torch.from_numpy(-2.0 * xh[:, 5])).numpy(), rtol=1e-12)
    assert (out[:, 13:] == 0).all() and (out[:, :10] == 0).all()


def test_calibration_rows_are_independent_and_bonus_enters_by_embedding():
    dims, W = _cal_model()
    m = oracle.Model(dims, W)
    r = rng(53)
    xh, lg = r.standard_normal((16, dims.d)), r.standard_normal((16, dims.vocab))
    base = oracle.calibrate(m, xh, 3, lg)
    xh2 = xh.copy()
    xh2[4] += 1.0
    out = oracle.calibrate(m, xh2, 3, lg)
    changed = np.abs(out - base).max(axis=1) > 1e-9
    assert changed[4] and not changed[np.arange(16) != 4].any()
    # two bonus tokens with equal embedding rows calibrate alike; a different row does not
    W2 = dict(W)
    emb = W["embed"].copy()
    emb[9] = emb[3]
    W2["embed"] = emb
    m2 = oracle.Model(dims, W2)
    np.testing.assert_array_equal(oracle.calibrate(m2, xh, 9, lg), oracle.calibrate(m2, xh, 3, lg))
    assert np.abs(oracle.calibrate(m, xh, 4, lg) - base).max() > 1e-6
