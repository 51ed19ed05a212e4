"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: hand-worked
values (tests/golden/hand_worked.json), closed forms, invariants the pages
state, brute force on tiny inputs, or special cases that reduce to a plain
formula. None of these tests needs a GPU.
"""
import json
import math
import os

import numpy as np
import pytest

from looped_ngpt_language_amd import synth
from oracle import (LAST_LOOP, PER_LOOP, OracleModel, attend, bf16_round, greedy, l2_normalize,
                    ngpt_residual, rope, self_speculative, self_speculative_reuse, silu)

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")))

# A deliberately non-square tiny shape: a transposed weight fails on shapes.
ODD = synth.ModelShape(d_model=24, n_heads=4, n_kv_heads=2, head_dim=8, d_ff=40, vocab=97,
                       n_in=2, n_rec=4, n_out=2, window=5, dtype=synth.F32)
# The pages' 8/20/8 stacks at toy width, for counts.
STACKS = synth.ModelShape(d_model=16, n_heads=2, n_kv_heads=1, head_dim=8, d_ff=24, vocab=61,
                          n_in=8, n_rec=20, n_out=8, window=4, dtype=synth.F32)


@pytest.fixture(scope="module")
def odd_weights():
    return synth.make_weights(ODD, seed=0, threads=2)


@pytest.fixture(scope="module")
def tiny_weights():
    return synth.make_weights(synth.TINY, seed=0, threads=4)


# ---------------------------------------------------------------- elementary

def test_l2_normalize_golden():
    for case in GOLDEN["l2_normalize"]:
        np.testing.assert_allclose(l2_normalize(case["v"]), case["expect"], rtol=0, atol=1e-15)


def test_l2_normalize_unit_and_zero():
    v = np.random.default_rng(5).standard_normal((7, 33))
    n = np.linalg.norm(l2_normalize(v), axis=-1)
    np.testing.assert_allclose(n, 1.0, atol=1e-14)
    with pytest.raises(FloatingPointError):
        l2_normalize(np.zeros(4))


def test_ngpt_residual_golden_and_limits():
    for case in GOLDEN["ngpt_residual"]:
        got = ngpt_residual(np.array(case["h"]), np.array(case["y"]), np.array(case["alpha"]))
        np.testing.assert_allclose(got, case["expect"], rtol=0, atol=1e-15)
    rng = np.random.default_rng(6)
    h = l2_normalize(rng.standard_normal((5, 16)))
    y = rng.standard_normal((5, 16))
    np.testing.assert_allclose(ngpt_residual(h, y, np.zeros(16)), h, atol=1e-15)        # alpha = 0
    np.testing.assert_allclose(ngpt_residual(h, y, np.ones(16)), l2_normalize(y), atol=1e-15)  # alpha = 1


def test_rope_golden():
    for case in GOLDEN["rope"]:
        x = np.array(case["x"], dtype=np.float64)[None, None, :]
        got = rope(x, np.array([case["pos"]]), case["theta"])[0, 0]
        np.testing.assert_allclose(got, case["expect"], rtol=0, atol=1e-15)


def test_rope_invariants():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 3, 32))
    k = rng.standard_normal((1, 3, 32))
    np.testing.assert_array_equal(rope(q, np.array([0]), 1e4), q)                  # position 0
    for p in (1, 17, 131071):
        np.testing.assert_allclose(np.linalg.norm(rope(q, np.array([p]), 1e4), axis=-1),
                                   np.linalg.norm(q, axis=-1), rtol=1e-13)       # norm kept
    # relative position: <R(q,m), R(k,n)> depends only on m - n
    def dot(m, n):
        return np.sum(rope(q, np.array([m]), 1e4) * rope(k, np.array([n]), 1e4), axis=-1)
    np.testing.assert_allclose(dot(10, 3), dot(107, 100), atol=1e-12)
    np.testing.assert_allclose(dot(5, 5), np.sum(q * k, axis=-1), atol=1e-12)


def test_silu_and_bf16_golden():
    np.testing.assert_allclose(silu(np.array(GOLDEN["silu"]["z"])), GOLDEN["silu"]["expect"], atol=1e-15)
    z = np.linspace(-6, 6, 25)
    np.testing.assert_allclose(silu(-z), silu(z) - z, atol=1e-14)   # silu(-z) = silu(z) - z
    b = GOLDEN["bf16_round"]
    np.testing.assert_array_equal(bf16_round(np.array(b["x"])), b["expect"])
    # every bf16 value is a fixed point; bf16 has 8 significant bits
    v = bf16_round(np.random.default_rng(1).standard_normal(1000))
    np.testing.assert_array_equal(bf16_round(v), v)
    m, _ = np.frexp(v)
    np.testing.assert_array_equal(m * 256, np.round(m * 256))


# ---------------------------------------------------------------- attention

def brute_attention(q, K, V, positions, window, H, Hk, scale):
    """Scalar triple loop with explicit exponentials (no vectorised softmax)."""
    T, dh = q.shape[0], q.shape[2]
    out = np.zeros((T, H, dh))
    for i in range(T):
        p = int(positions[i])
        for h in range(H):
            g = h * Hk // H
            keys = [j for j in range(p + 1) if window is None or j > p - window]
            sc = [scale * sum(q[i, h, e] * K[j, g, e] for e in range(dh)) for j in keys]
            mx = max(sc)
            w = [math.exp(s - mx) for s in sc]
            tot = sum(w)
            for e in range(dh):
                out[i, h, e] = sum(w[a] * V[j, g, e] for a, j in enumerate(keys)) / tot
    return out


@pytest.mark.parametrize("window", [None, 1, 3, 100])
def test_attention_brute_force(window):
    rng = np.random.default_rng(11)
    L, H, Hk, dh = 9, 4, 2, 5
    K = rng.standard_normal((L, Hk, dh))
    V = rng.standard_normal((L, Hk, dh))
    pos = np.array([2, 5, 6, 8])
    q = rng.standard_normal((4, H, dh))
    got = attend(q, K, V, pos, window, H, Hk, 1.7)
    np.testing.assert_allclose(got, brute_attention(q, K, V, pos, window, H, Hk, 1.7), atol=1e-13)


def test_attention_golden_two_keys():
    g = GOLDEN["attention_two_keys"]
    q = np.array(g["q"])[:, None, :]
    K = np.array(g["k"])[:, None, :]
    V = np.array(g["v"])[:, None, :]
    pos = np.array([0, 1])
    np.testing.assert_allclose(attend(q, K, V, pos, None, 1, 1, g["scale"])[:, 0], g["expect_full"], atol=1e-15)
    np.testing.assert_allclose(attend(q, K, V, pos, 1, 1, 1, g["scale"])[:, 0], g["expect_window1"], atol=1e-15)


def test_attention_special_cases():
    rng = np.random.default_rng(12)
    L, H, Hk, dh = 12, 6, 3, 4
    K = rng.standard_normal((L, Hk, dh))
    V = rng.standard_normal((L, Hk, dh))
    pos = np.arange(L)
    q = rng.standard_normal((L, H, dh))
    full = attend(q, K, V, pos, None, H, Hk, 2.0)
    np.testing.assert_allclose(attend(q, K, V, pos, L, H, Hk, 2.0), full, atol=1e-15)       # W >= T is full
    w1 = attend(q, K, V, pos, 1, H, Hk, 2.0)
    np.testing.assert_allclose(w1, V[:, np.arange(H) // (H // Hk), :], atol=1e-15)        # W = 1 gives v_i
    Kc = np.ones((L, Hk, dh))                                                              # equal scores
    mean = np.cumsum(V, axis=0) / np.arange(1, L + 1)[:, None, None]
    np.testing.assert_allclose(attend(q, Kc, V, pos, None, H, Hk, 2.0),
                               mean[:, np.arange(H) // (H // Hk), :], atol=1e-13)
    # GQA mapping: heads 0,1 -> kv 0, heads 2,3 -> kv 1, heads 4,5 -> kv 2
    Vg = np.zeros((L, Hk, dh))
    for g in range(Hk):
        Vg[:, g, :] = g + 1
    out = attend(q, K, Vg, pos, None, H, Hk, 2.0)
    np.testing.assert_allclose(out[:, :, 0], np.tile([1, 1, 2, 2, 3, 3], (L, 1)), atol=1e-14)
    # H_kv = H is plain multi-head attention: equal to running each head alone
    Km = rng.standard_normal((L, H, dh))
    Vm = rng.standard_normal((L, H, dh))
    mha = attend(q, Km, Vm, pos, 5, H, H, 2.0)
    for h in range(H):
        one = attend(q[:, h:h + 1], Km[:, h:h + 1], Vm[:, h:h + 1], pos, 5, 1, 1, 2.0)
        np.testing.assert_allclose(mha[:, h], one[:, 0], atol=1e-15)


# ---------------------------------------------------------------- block / loop

def test_single_token_block_reduces_to_value_path(odd_weights):
    """With one token every query sees only its own key, so attention returns v of its KV
    head: block(h) = MLP-step(N(h + a_A*(N(W_o [v_g(h)]) - h))). Pins W_v/W_o orientation,
    the GQA map and both residual steps without RoPE or softmax."""
    s = ODD
    m = OracleModel(s, odd_weights, PER_LOOP, 1)
    from oracle.model import _Seq
    seq = _Seq(s.n_kv_heads, s.head_dim)
    W = m.blocks[1]
    h = l2_normalize(np.random.default_rng(3).standard_normal((1, s.d_model)))
    got = m._block(h, 1, 1, seq, np.array([0]))
    v = (h @ W["wv"].T).reshape(s.n_kv_heads, s.head_dim)
    o = np.concatenate([v[hq * s.n_kv_heads // s.n_heads] for hq in range(s.n_heads)])
    y = W["wo"] @ o
    h1 = h[0] + W["alpha_attn"] * (y / np.linalg.norm(y) - h[0])
    h1 = h1 / np.linalg.norm(h1)
    g = W["wg"] @ h1
    y2 = W["wd"] @ ((g / (1 + np.exp(-g))) * (W["wu"] @ h1))
    h2 = h1 + W["alpha_mlp"] * (y2 / np.linalg.norm(y2) - h1)
    np.testing.assert_allclose(got[0], h2 / np.linalg.norm(h2), atol=1e-13)


def test_two_token_block_query_key_path(odd_weights):
    """Second token: attention weights are the softmax of scale * N(RoPE(W_q h1)).N(RoPE(W_k h_j))
    over j = 0, 1 (window 5 covers both). Checked head by head against explicit rotations."""
    s = ODD
    m = OracleModel(s, odd_weights, PER_LOOP, 1)
    from oracle.model import _Seq
    seq = _Seq(s.n_kv_heads, s.head_dim)
    W = m.blocks[0]
    h = l2_normalize(np.random.default_rng(4).standard_normal((2, s.d_model)))
    got = m._block(h, 0, 1, seq, np.array([0, 1]))
    dh, half = s.head_dim, s.head_dim // 2

    def rot(x, p):
        out = np.empty(dh)
        for i in range(half):
            a = p * s.rope_theta ** (-2 * i / dh)
            out[i] = x[i] * math.cos(a) - x[i + half] * math.sin(a)
            out[i + half] = x[i] * math.sin(a) + x[i + half] * math.cos(a)
        return out / np.linalg.norm(out)
    q = (W["wq"] @ h[1]).reshape(s.n_heads, dh)
    ks = [(W["wk"] @ h[j]).reshape(s.n_kv_heads, dh) for j in range(2)]
    vs = [(W["wv"] @ h[j]).reshape(s.n_kv_heads, dh) for j in range(2)]
    o = []
    for hq in range(s.n_heads):
        g = hq * s.n_kv_heads // s.n_heads
        sc = [s.scale * rot(q[hq], 1) @ rot(ks[j][g], j) for j in range(2)]
        w1 = 1.0 / (1.0 + math.exp(sc[0] - sc[1]))
        o.append((1 - w1) * vs[0][g] + w1 * vs[1][g])
    y = W["wo"] @ np.concatenate(o)
    h1 = h[1] + W["alpha_attn"] * (y / np.linalg.norm(y) - h[1])
    h1 = h1 / np.linalg.norm(h1)
    g = W["wg"] @ h1
    y2 = W["wd"] @ ((g / (1 + np.exp(-g))) * (W["wu"] @ h1))
    h2 = h1 + W["alpha_mlp"] * (y2 / np.linalg.norm(y2) - h1)
    np.testing.assert_allclose(got[1], h2 / np.linalg.norm(h2), atol=1e-13)


def plain_stack(m, tokens):
    """The ordinary non-looped model: every physical block once, in order."""
    from oracle.model import _Seq
    seq = _Seq(m.s.n_kv_heads, m.s.head_dim)
    pos = np.arange(len(tokens))
    h = m.E[np.asarray(tokens)]
    for j in range(m.s.n_blocks):
        h = m._block(h, j, 1, seq, pos)
    return h


@pytest.mark.parametrize("mode", [PER_LOOP, LAST_LOOP])
def test_k1_is_plain_stack(tiny_weights, mode):
    toks = synth.prompt_tokens(synth.TINY, 12)
    m = OracleModel(synth.TINY, tiny_weights, mode, 1)
    m.prefill(0, toks, 12)
    np.testing.assert_allclose(m.last_hidden, plain_stack(m, toks), atol=1e-13)


def test_loop_states_follow_update(tiny_weights):
    """x, u_t, s_t are unit norm; u_1 = x; u_t = N(s_{t-1} + x) for t >= 2."""
    toks = synth.prompt_tokens(synth.TINY, 10)
    m = OracleModel(synth.TINY, tiny_weights, PER_LOOP, 4)
    tr = {}
    m.prefill(0, toks, 1, trace=tr)
    x = tr["x"]
    np.testing.assert_allclose(np.linalg.norm(x, axis=-1), 1, atol=1e-14)
    for t in range(4):
        np.testing.assert_allclose(np.linalg.norm(tr["u"][t], axis=-1), 1, atol=1e-14)
        np.testing.assert_allclose(np.linalg.norm(tr["s"][t], axis=-1), 1, atol=1e-14)
    np.testing.assert_allclose(tr["u"][0], x, atol=1e-15)
    for t in range(1, 4):
        want = tr["s"][t - 1] + x
        np.testing.assert_allclose(tr["u"][t], want / np.linalg.norm(want, axis=-1, keepdims=True), atol=1e-15)
        assert np.max(np.abs(tr["s"][t] - tr["s"][t - 1])) > 1e-3   # the core actually runs again
    np.testing.assert_allclose(np.linalg.norm(m.last_hidden, axis=-1), 1, atol=1e-14)


@pytest.mark.parametrize("k", [1, 2, 4])
def test_application_counts(k):
    ref = GOLDEN["layer_applications"]
    w = synth.make_weights(STACKS, seed=0, threads=2)
    m = OracleModel(STACKS, w, PER_LOOP, k)
    m.prefill(0, [1], 1)
    assert m.counts["block"] == ref["blocks"][str(k)]
    assert m.counts["sublayer"] == ref["sublayers"][str(k)]
    assert m.counts["full"] == ref["full"][str(k)]
    assert m.counts["swa"] == ref["swa"][str(k)]
    slots = GOLDEN["kv_slots"]
    assert m.n_slots() == slots["per_loop"][str(k)]
    assert len(m.seqs[0].K) == slots["per_loop"][str(k)]
    m2 = OracleModel(STACKS, w, LAST_LOOP, k)
    m2.prefill(0, [1], 1)
    assert m2.n_slots() == slots["last_loop"][str(k)]
    assert len(m2.seqs[0].K) == slots["last_loop"][str(k)]


# ---------------------------------------------------------------- KV modes

def run_greedy(w, mode, k, toks, n):
    m = OracleModel(synth.TINY, w, mode, k)
    ids, lg = greedy(m, 0, toks, n)
    return ids, lg


def test_modes_identical_at_k1(tiny_weights):
    toks = synth.prompt_tokens(synth.TINY, 20)
    a = run_greedy(tiny_weights, PER_LOOP, 1, toks, 6)
    b = run_greedy(tiny_weights, LAST_LOOP, 1, toks, 6)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


@pytest.mark.parametrize("k", [2, 4])
def test_modes_identical_for_whole_prompt_prefill(tiny_weights, k):
    toks = synth.prompt_tokens(synth.TINY, 24)
    ma = OracleModel(synth.TINY, tiny_weights, PER_LOOP, k)
    mb = OracleModel(synth.TINY, tiny_weights, LAST_LOOP, k)
    la, _ = ma.prefill(0, toks, 24)
    lb, _ = mb.prefill(0, toks, 24)
    np.testing.assert_array_equal(la, lb)
    # single-token prompt
    ma.prefill(1, toks[:1], 1)
    mb.prefill(1, toks[:1], 1)
    np.testing.assert_array_equal(ma.last_hidden, mb.last_hidden)


@pytest.mark.parametrize("k", [2, 4])
def test_modes_differ_in_decode(tiny_weights, k):
    """Last-loop decode: earlier-loop queries read the final loop's KV, so results differ."""
    toks = synth.prompt_tokens(synth.TINY, 20)
    a = run_greedy(tiny_weights, PER_LOOP, k, toks, 3)
    b = run_greedy(tiny_weights, LAST_LOOP, k, toks, 3)
    np.testing.assert_array_equal(a[1][0], b[1][0])          # prefill row identical
    assert np.max(np.abs(a[1][1:] - b[1][1:])) > 1e-6        # decode rows differ


def test_per_loop_chunking_invariance(tiny_weights):
    toks = synth.prompt_tokens(synth.TINY, 21)
    whole = OracleModel(synth.TINY, tiny_weights, PER_LOOP, 2)
    lw, _ = whole.prefill(0, toks, 21)
    one = OracleModel(synth.TINY, tiny_weights, PER_LOOP, 2)
    rows = [one.prefill(0, toks[i:i + 1], 1)[0][0] for i in range(21)]
    np.testing.assert_allclose(np.array(rows), lw, atol=1e-13)
    ch = OracleModel(synth.TINY, tiny_weights, PER_LOOP, 2)
    out = []
    for a, b in ((0, 5), (5, 6), (6, 17), (17, 21)):
        out.append(ch.prefill(0, toks[a:b], b - a)[0])
    np.testing.assert_allclose(np.concatenate(out), lw, atol=1e-13)


def test_sliding_window_binds(tiny_weights):
    """Changing a token outside every sliding window but inside the full layers' reach changes
    the output (full layers see it); with all layers sliding it would not."""
    toks = synth.prompt_tokens(synth.TINY, 40)
    m = OracleModel(synth.TINY, tiny_weights, PER_LOOP, 1)
    l1, _ = m.prefill(0, toks, 1)
    t2 = toks.copy()
    t2[0] = (t2[0] + 1) % synth.TINY.vocab
    m2 = OracleModel(synth.TINY, tiny_weights, PER_LOOP, 1)
    l2, _ = m2.prefill(0, t2, 1)
    assert np.max(np.abs(l1 - l2)) > 0
    no_full = synth.TINY.replace(full_every=10**6)
    m3 = OracleModel(no_full, tiny_weights, PER_LOOP, 1)
    m4 = OracleModel(no_full, tiny_weights, PER_LOOP, 1)
    # receptive field of 8 sliding layers of window 16 over the last row: 8*15 = 120 > 40, so
    # shorten the window to make token 0 unreachable: 8 * (4-1) = 24 < 39
    m3.s = m4.s = no_full.replace(window=4)
    a, _ = m3.prefill(0, toks, 1)
    b, _ = m4.prefill(0, t2, 1)
    np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------- spec decoding / errors

def test_self_speculative_per_loop_equals_k4_greedy(tiny_weights):
    toks = synth.prompt_tokens(synth.TINY, 16)
    ref, _ = run_greedy(tiny_weights, PER_LOOP, 4, toks, 12)
    m = OracleModel(synth.TINY, tiny_weights, PER_LOOP, 4)
    got = self_speculative(m, 0, toks, 13)
    np.testing.assert_array_equal(got[:13], ref[:13])


@pytest.mark.parametrize("mode", [PER_LOOP, LAST_LOOP])
def test_spec_reuse_round_equals_plain_verify(tiny_weights, mode):
    """One draft/verify round both ways: the verify logits of the reuse procedure (input stack and
    loop 1 of drafted rows taken from the k = 1 draft, cache kept) equal those of a fresh verify
    chunk, to fp64 rounding."""
    toks = synth.prompt_tokens(synth.TINY, 20)
    gamma = 4
    ma = OracleModel(synth.TINY, tiny_weights, mode, 4)
    mb = OracleModel(synth.TINY, tiny_weights, mode, 4)
    _, ida = ma.prefill(0, toks, 1)
    mb.prefill(0, toks, 1)
    last = int(ida[0])
    base = ma.seq_len(0)
    # plain: draft at k = 1, truncate, verify [last, d1..d4] at k = 4
    ma.set_loops(1)
    drafts, tok = [], last
    for _ in range(gamma):
        _, i = ma.decode([0], [tok])
        tok = int(i[0])
        drafts.append(tok)
    ma.truncate(0, base)
    ma.set_loops(4)
    la, _ = ma.prefill(0, [last] + drafts, gamma + 1)
    # reuse: same drafts, x and s_1 kept, loops 2..4 + output stack for all rows
    mb.set_loops(1)
    xs, s1s = [], []
    for t in [last] + drafts[:-1]:
        tr = {}
        mb.prefill(0, [t], 1, trace=tr)
        xs.append(tr["x"][0])
        s1s.append(tr["s"][0][0])
    xl, s1l = mb.head_rows(0, [drafts[-1]])
    mb.set_loops(4)
    lb, _ = mb.resume_rows(0, base, np.array(xs + [xl[0]]), np.array(s1s + [s1l[0]]), gamma + 1)
    assert np.max(np.abs(la - lb)) < 1e-9
    assert ma.seq_len(0) == mb.seq_len(0) == base + gamma + 1


@pytest.mark.parametrize("mode", [PER_LOOP, LAST_LOOP])
@pytest.mark.parametrize("gamma", [2, 4])
def test_spec_reuse_ids_equal_plain_spec(tiny_weights, mode, gamma):
    toks = synth.prompt_tokens(synth.TINY, 16)
    a = self_speculative(OracleModel(synth.TINY, tiny_weights, mode, 4), 0, toks, 14, gamma=gamma, k_draft=1)
    b = self_speculative_reuse(OracleModel(synth.TINY, tiny_weights, mode, 4), 0, toks, 14, gamma=gamma)
    np.testing.assert_array_equal(a[:14], b[:14])
    if mode == PER_LOOP:                          # and both equal plain k = 4 greedy
        ref, _ = run_greedy(tiny_weights, PER_LOOP, 4, toks, 13)
        np.testing.assert_array_equal(b[:14], ref[:14])


def test_error_paths(tiny_weights):
    m = OracleModel(synth.TINY, tiny_weights, PER_LOOP, 2)
    for bad in (0, 5, -1):
        with pytest.raises(ValueError):
            m.set_loops(bad)
    m.prefill(0, [1, 2, 3], 1)
    with pytest.raises(RuntimeError):
        m.set_kv_mode(LAST_LOOP)
    m.set_loops(4)
    with pytest.raises(RuntimeError):             # per-loop cache holds only 2 loops
        m.decode([0], [5])
    m.set_loops(1)
    m.decode([0], [5])
    with pytest.raises(ValueError):
        m.truncate(0, 10)
    m.release(0)
    m.set_kv_mode(LAST_LOOP)
    m.set_loops(4)
    m.prefill(0, [1, 2, 3], 1)
    m.set_loops(1)
    m.decode([0], [4])
    m.set_loops(4)
    m.decode([0], [4])                            # last-loop: any loop count reads slot j


def test_bf16_storage_points():
    """bf16 shapes: cache rows are bf16-exact; the result stays close to the unrounded model."""
    s16 = ODD.replace(dtype=synth.BF16)
    w = synth.make_weights(s16, seed=0, threads=2)
    toks = synth.prompt_tokens(s16, 9)
    m16 = OracleModel(s16, w, PER_LOOP, 2)
    l16, _ = m16.prefill(0, toks, 9)
    for sl in m16.seqs[0].K:
        K = m16.seqs[0].K[sl][:9]
        np.testing.assert_array_equal(bf16_round(K), K)
        np.testing.assert_array_equal(bf16_round(m16.seqs[0].V[sl][:9]), m16.seqs[0].V[sl][:9])
    m32 = OracleModel(s16.replace(dtype=synth.F32), w, PER_LOOP, 2)
    l32, _ = m32.prefill(0, toks, 9)
    d = np.max(np.abs(l16 - l32))
    assert 0 < d < 2e-2
