"""Pins for the oracle's sampling path (CPU only).

Each test checks the oracle against something other than itself: a library
routine in a special case, a closed form, exhaustive enumeration, a
statistical law, or the gold tests the dormouse verification page proposes
(section 7: the off-by-one gate, Eq 6 against a hand-stepped three-position
reference, the width of the confidence input).
"""
import itertools
import math

import numpy as np
import pytest
from scipy import special, stats

import synth


def small(V=16, r=4, d=8, gamma=3, B=5, dtype="f32", head="markov", seed=11, **kw):
    base = dict(u_std=2.0, h_std=1.0, w1_std=0.5, w2_std=0.5, wconf_std=0.3,
                wrnn_std=0.5, anchors="uniform", temperature=1.0)
    base.update(kw)
    return synth.make_inputs(V=V, r=r, d=d, gamma=gamma, B=B, dtype=dtype, head=head,
                             seed=seed, **base)


def f64(inp, a):
    return inp.as_f32(a).astype(np.float64)


# ---------------------------------------------------------------- Eq 4 / 5

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_w2_reduces_to_softmax_of_base_logits(oracle_lib, dtype):
    # Eq 4 with B_k = 0 is p_k = softmax(U_k): logp must equal a library
    # log-softmax of U at the sampled token, and greedy must be argmax U_k.
    inp = small(V=50, dtype=dtype, B=6, gamma=4)
    inp.W2 = np.zeros_like(inp.W2)
    U = f64(inp, inp.U)
    out = oracle_lib.draft_block(inp, seed=3)
    ls = special.log_softmax(U, axis=-1)
    for b in range(inp.B):
        for k in range(inp.gamma):
            x = out["tokens"][b, k]
            assert abs(out["logp"][b, k] - ls[b, k, x]) < 1e-12
    greedy = oracle_lib.draft_block(inp, temperature=np.zeros(inp.B, np.float32))
    assert np.array_equal(greedy["tokens"], np.argmax(U, axis=-1))


def test_markov_bias_is_embedding_times_projection(oracle_lib):
    # Eq 5: with the previous token fixed, logp of the sampled token equals a
    # library log-softmax of U_k + W1[prev] @ W2 (matrix product by numpy).
    inp = small(V=40, r=6, B=3, gamma=4)
    out = oracle_lib.draft_block(inp, seed=9)
    U, W1, W2 = f64(inp, inp.U), f64(inp, inp.W1), f64(inp, inp.W2)
    for b in range(inp.B):
        prev = inp.anchor[b]
        for k in range(inp.gamma):
            z = U[b, k] + W1[prev] @ W2
            x = out["tokens"][b, k]
            assert abs(out["logp"][b, k] - special.log_softmax(z)[x]) < 1e-11
            prev = x


@pytest.mark.parametrize("head", ["markov", "rnn"])
def test_block_probabilities_sum_to_one_exhaustive(oracle_lib, head):
    # Eq 4 is a product of conditionals, so over all V^gamma blocks it sums to 1.
    V, gamma = 4, 3
    inp = small(V=V, r=3, d=5, gamma=gamma, B=1, head=head, w1_std=1.0, w2_std=1.0)
    blocks = np.array(list(itertools.product(range(V), repeat=gamma)), np.int32)
    n = len(blocks)
    rep = _replicate(inp, n)
    lp = oracle_lib.block_logprob(rep, blocks)
    assert abs(np.exp(lp).sum() - 1.0) < 1e-12


def _replicate(inp, n):
    """The same single block repeated n times (shared anchor, U, h)."""
    rep = synth.Inputs(**{f: getattr(inp, f) for f in inp.__dataclass_fields__})
    rep.B = n
    rep.anchor = np.repeat(inp.anchor[:1], n)
    rep.U = np.ascontiguousarray(np.repeat(inp.U[:1], n, axis=0))
    rep.h = np.ascontiguousarray(np.repeat(inp.h[:1], n, axis=0))
    rep.temperature = np.repeat(inp.temperature[:1], n)
    return rep


@pytest.mark.parametrize("head,temp", [("markov", 1.0), ("rnn", 1.0), ("markov", 2.0)])
def test_sampler_law_matches_block_probabilities(oracle_lib, head, temp):
    # Gumbel-max draws x_k from softmax(z_k / T): the frequencies of many
    # sampled blocks must follow the exact Eq 4 product (chi-square, fixed seed).
    V, gamma, n = 4, 3, 120_000
    inp = small(V=V, r=3, d=5, gamma=gamma, B=1, head=head, w1_std=1.0, w2_std=1.0,
                u_std=1.0, temperature=temp)
    rep = _replicate(inp, n)
    out = oracle_lib.draft_block(rep, seed=2024)
    codes = (out["tokens"] * np.array([V * V, V, 1])).sum(axis=1)
    counts = np.bincount(codes, minlength=V**gamma)
    blocks = np.array(list(itertools.product(range(V), repeat=gamma)), np.int32)
    probs = np.exp(oracle_lib.block_logprob(_replicate(inp, len(blocks)), blocks))
    assert abs(probs.sum() - 1) < 1e-12
    expected = probs * n
    keep = expected > 5
    chi2 = (((counts - expected) ** 2) / expected)[keep].sum()
    p = stats.chi2.sf(chi2, keep.sum() - 1)
    assert p > 1e-3, (chi2, p)
    # logp of each sampled block equals the Eq 4 log-probability of that block
    lp = oracle_lib.block_logprob(_replicate(inp, 50), out["tokens"][:50])
    assert np.allclose(out["logp"][:50].sum(axis=1), lp, atol=1e-12)


def test_toy_phrase_coupling(oracle_lib):
    # The "no problem" / "of course" picture (mainlymatmul page, "The problem
    # with parallel generation" and "A parallel backbone with autoregressive
    # sampling"): tokens 0 "no", 1 "of", 2 "problem", 3 "course".  Base logits
    # split evenly over {no, of} then {problem, course}.  With no transition
    # bias the four pairs are equally likely; a bigram bias favouring
    # no->problem and of->course moves the mass onto the two coherent pairs.
    V, gamma = 4, 2
    big = 30.0
    inp = small(V=V, r=2, d=1, gamma=gamma, B=1)
    inp.U = np.array([[[big, big, 0, 0], [0, 0, big, big]]], np.float32)
    inp.anchor = np.array([3], np.int32)
    inp.W1 = np.zeros((V, 2), np.float32)
    inp.W2 = np.zeros((2, V), np.float32)
    pairs = np.array([[0, 2], [0, 3], [1, 2], [1, 3]], np.int32)
    rep = _replicate(inp, 4)
    p_flat = np.exp(oracle_lib.block_logprob(rep, pairs))
    assert np.allclose(p_flat, 0.25, atol=1e-12)
    inp.W1[0] = [1, 0]
    inp.W1[1] = [0, 1]
    inp.W2[0] = [0, 0, 2, -2]   # after "no": favour "problem"
    inp.W2[1] = [0, 0, -2, 2]   # after "of": favour "course"
    p_bigram = np.exp(oracle_lib.block_logprob(_replicate(inp, 4), pairs))
    coherent = 0.5 / (1 + math.exp(-4))  # each: 1/2 * sigmoid(4)
    assert np.allclose(p_bigram, [coherent, 0.5 - coherent, 0.5 - coherent, coherent], atol=1e-12)


# ---------------------------------------------------------------- Eq 7

def test_zero_confidence_weights_give_half(oracle_lib):
    inp = small(B=4, gamma=6)
    inp.w_conf = np.zeros_like(inp.w_conf)
    out = oracle_lib.draft_block(inp)
    assert np.all(out["conf"] == 0.5)
    assert np.all(out["surv"] == 0.5 ** np.arange(1, 7)[None, :])


def test_confidence_reads_hidden_and_previous_token_embedding(oracle_lib):
    # Width check (dormouse page, section 7 item 3, delta-table row D9): the
    # confidence input is [h_k; W1[x_{k-1}]] of width d + r, h part first.
    inp = small(V=30, r=5, d=7, B=3, gamma=4)
    out = oracle_lib.draft_block(inp, seed=1)
    h, W1, w = f64(inp, inp.h), f64(inp, inp.W1), f64(inp, inp.w_conf)
    assert w.shape == (inp.d + inp.r,)
    for b in range(inp.B):
        prev = inp.anchor[b]
        S = 1.0
        for k in range(inp.gamma):
            c = special.expit(w[: inp.d] @ h[b, k] + w[inp.d:] @ W1[prev])
            S *= c
            assert abs(out["conf"][b, k] - c) < 1e-14
            assert abs(out["surv"][b, k] - S) < 1e-14
            prev = out["tokens"][b, k]


def _identity_encoded(V, r, d, gamma, B, dtype="f32"):
    """W1 row v carries v/128 in column 0 and the confidence weights read only
    that column, so c_k = sigmoid(prev/128) reveals which token was gathered."""
    inp = small(V=V, r=r, d=d, gamma=gamma, B=B, dtype=dtype)
    W1 = np.zeros((V, r), np.float32)
    W1[:, 0] = np.arange(V) / 128.0
    w = np.zeros(d + r, np.float32)
    w[d] = 1.0
    if dtype == "bf16":
        inp.W1, inp.w_conf = synth.f32_to_bf16_bits(W1), synth.f32_to_bf16_bits(w)
    else:
        inp.W1, inp.w_conf = W1, w
    return inp


def test_off_by_one_gate_sampling(oracle_lib):
    # dormouse page, section 7 item 1 (adapted to sampling): the token fed at
    # step k is x_{k-1}, the anchor at k = 1.  Exact, not a tolerance test.
    inp = _identity_encoded(V=64, r=2, d=3, gamma=5, B=6)
    out = oracle_lib.draft_block(inp, seed=5)
    prev = np.concatenate([inp.anchor[:, None], out["tokens"][:, :-1]], axis=1)
    fed = np.rint(special.logit(out["conf"]) * 128).astype(int)
    assert np.array_equal(fed, prev)


def test_forced_prefix_conditioning(oracle_lib):
    inp = small(V=40, B=4, gamma=5)
    own = oracle_lib.draft_block(inp, seed=8)
    again = oracle_lib.draft_block(inp, seed=8, forced_prev=own["tokens"])
    for key in ("tokens", "logp", "conf", "surv", "gap"):
        assert np.array_equal(own[key], again[key])
    # a forced prefix is what the next step conditions on
    forced = (own["tokens"] + 1) % inp.V
    f = oracle_lib.draft_block(inp, seed=8, forced_prev=forced)
    # the last step's logp is the Eq 4 conditional given the forced prefix:
    # log P(forced[:-1], x) - log P(forced[:-1])
    blk = forced.copy()
    blk[:, -1] = f["tokens"][:, -1]
    lp_full = oracle_lib.block_logprob(inp, blk)
    lp_prefix = oracle_lib.block_logprob(_truncate(inp, inp.gamma - 1), blk[:, :-1])
    assert np.allclose(lp_full - lp_prefix, f["logp"][:, -1], atol=1e-12)


def _truncate(inp, g):
    t = synth.Inputs(**{f: getattr(inp, f) for f in inp.__dataclass_fields__})
    t.gamma = g
    t.U = np.ascontiguousarray(inp.U[:, :g])
    t.h = np.ascontiguousarray(inp.h[:, :g])
    return t


def test_gap_and_runner_up(oracle_lib):
    inp = small(V=20, B=3, gamma=3)
    out = oracle_lib.draft_block(inp, temperature=np.zeros(3, np.float32))
    U, W1, W2 = f64(inp, inp.U), f64(inp, inp.W1), f64(inp, inp.W2)
    for b in range(3):
        prev = inp.anchor[b]
        for k in range(3):
            z = U[b, k] + W1[prev] @ W2
            order = np.argsort(-z, kind="stable")
            assert out["tokens"][b, k] == order[0]
            assert out["second"][b, k] == order[1]
            assert abs(out["gap"][b, k] - (z[order[0]] - z[order[1]])) < 1e-12
            prev = order[0]


def test_lowest_index_wins_ties(oracle_lib):
    inp = small(V=12, B=1, gamma=2)
    inp.U = np.zeros_like(inp.U)
    inp.U[0, :, [3, 7, 9]] = 5.0
    inp.W2 = np.zeros_like(inp.W2)
    out = oracle_lib.draft_block(inp, temperature=np.zeros(1, np.float32))
    assert out["tokens"].tolist() == [[3, 3]]


# ---------------------------------------------------------------- Eq 6

def test_rnn_three_position_hand_reference(oracle_lib):
    # dormouse page, section 7 item 2: Eq 6 stepped by hand over three
    # positions with s_0 = 0.  r = d = 1, V = 2.  The joint projection's rows
    # are (gate, candidate, output); its columns (s, e, h).
    #   gate row [0, 0, a]  -> g_k = sigmoid(a h_k)
    #   cand row [0, 0, 1]  -> c~_k = tanh(h_k)
    #   out  row [1, 0, 0]  -> o_k = tanh(s_{k-1})
    # W2 = [[1, 0]] so z_k = U_k + (o_k, 0); U = 0 so p_k(0) = sigmoid(o_k).
    a = 0.7
    hs = [0.9, -1.3, 2.1]
    inp = small(V=2, r=1, d=1, gamma=3, B=1, head="rnn")
    inp.U = np.zeros((1, 3, 2), np.float32)
    inp.h = np.array(hs, np.float32).reshape(1, 3, 1)
    inp.W1 = np.array([[0.25], [-0.5]], np.float32)
    inp.W2 = np.array([[1.0, 0.0]], np.float32)
    inp.W_rnn = np.array([[0, 0, a], [0, 0, 1], [1, 0, 0]], np.float32)
    hs32 = [float(np.float32(x)) for x in hs]
    a32 = float(np.float32(a))
    s, o = 0.0, []
    for k in range(3):
        o.append(math.tanh(s))
        g = 1 / (1 + math.exp(-a32 * hs32[k]))
        s = g * s + (1 - g) * math.tanh(hs32[k])
    blocks = np.array([[0, 0, 0], [1, 1, 1], [0, 1, 0]], np.int32)
    lp = oracle_lib.block_logprob(_replicate(inp, 3), blocks)
    logsig = lambda t: -math.log1p(math.exp(-t))
    want = [sum(logsig(ok) for ok in o),
            sum(logsig(-ok) for ok in o),
            logsig(o[0]) + logsig(-o[1]) + logsig(o[2])]
    assert np.allclose(lp, want, atol=1e-13)
    assert o[0] == 0.0 and o[1] != 0.0


def test_rnn_zero_output_rows_equal_markov_without_bias(oracle_lib):
    inp = small(V=30, r=4, d=6, B=3, gamma=4, head="rnn")
    inp.W_rnn[2 * inp.r:] = 0.0
    rnn = oracle_lib.draft_block(inp, seed=4)
    mk = synth.Inputs(**{f: getattr(inp, f) for f in inp.__dataclass_fields__})
    mk.head = "markov"
    mk.W2 = np.zeros_like(inp.W2)
    markov = oracle_lib.draft_block(mk, seed=4)
    for key in ("tokens", "logp", "conf", "surv"):
        assert np.array_equal(rnn[key], markov[key])


def test_rnn_zero_candidate_keeps_state_zero(oracle_lib):
    # W_c = 0 => c~ = 0 => s_k = g s_{k-1} = 0 for all k, so the s-columns of
    # the projection can be zeroed without changing anything.
    inp = small(V=30, r=4, d=6, B=3, gamma=4, head="rnn")
    r = inp.r
    inp.W_rnn[r:2 * r] = 0.0
    a = oracle_lib.draft_block(inp, seed=6)
    inp2 = synth.Inputs(**{f: getattr(inp, f) for f in inp.__dataclass_fields__})
    inp2.W_rnn = inp.W_rnn.copy()
    inp2.W_rnn[:, :r] = 0.0
    b = oracle_lib.draft_block(inp2, seed=6)
    for key in ("tokens", "logp"):
        assert np.array_equal(a[key], b[key])
    # and with W_c != 0 the state matters (the s-columns change the result)
    inp3 = small(V=30, r=4, d=6, B=3, gamma=4, head="rnn")
    c = oracle_lib.draft_block(inp3, seed=6)
    inp4 = synth.Inputs(**{f: getattr(inp3, f) for f in inp3.__dataclass_fields__})
    inp4.W_rnn = inp3.W_rnn.copy()
    inp4.W_rnn[:, :r] = 0.0
    d = oracle_lib.draft_block(inp4, seed=6)
    assert not np.allclose(c["logp"][:, 1:], d["logp"][:, 1:])
    assert np.array_equal(c["logp"][:, 0], d["logp"][:, 0])  # s_0 = 0


def test_threads_do_not_change_results(oracle_lib):
    inp = small(V=64, B=9, gamma=4, head="rnn")
    a = oracle_lib.draft_block(inp, seed=1, nthreads=1)
    b = oracle_lib.draft_block(inp, seed=1, nthreads=4)
    for key in a:
        assert np.array_equal(a[key], b[key])


def test_rejects_out_of_range_anchor(oracle_lib):
    inp = small(V=10, B=2)
    inp.anchor = np.array([3, 10], np.int32)
    with pytest.raises(ValueError):
        oracle_lib.draft_block(inp)
