"""Pins of the oracle's verification step (trim, accept/reject, final draw).

What the pages fix about it: the target checks the drafted block and keeps
the leading tokens up to the first rejection, and the result is still the
target's distribution (bowenzhou "Why DSpark?"); c* = 1 - TV(p_d, p_t) is the
single-step acceptance probability of the standard accept/reject rule
(Meridian section 3); pruning by confidence cuts a suffix and the kept tokens
are verified as usual (bowenzhou "设计", "Results").  Pinned here:
  - the first and second emitted tokens follow the target's distribution at
    their positions (chi-square over many independent blocks), while the
    drafter's own first token measurably does not (the test's power);
  - the first-position acceptance frequency equals 1 - TV(p_d, p_t);
  - after trimming every position away the emitted token still follows the
    target;
  - greedy verification keeps exactly the leading tokens that equal the
    target's argmax and then emits that argmax;
  - a target equal to the drafter accepts every token.
"""
import numpy as np
import pytest
from scipy import stats
from scipy.special import softmax

import oracle
import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def tiny(B=20000, V=5, gamma=2, seed=5, temperature=1.0):
    inp = synth.make_inputs(V=V, r=4, d=3, gamma=gamma, B=1, dtype="f32", head="markov", seed=seed,
                            u_std=1.0, w1_std=0.8, w2_std=0.8, anchors="uniform",
                            temperature=temperature)
    # B copies of one block: identical inputs, independent noise per block
    inp.U = np.ascontiguousarray(np.repeat(inp.U, B, axis=0))
    inp.h = np.ascontiguousarray(np.repeat(inp.h, B, axis=0))
    inp.anchor = np.repeat(inp.anchor, B)
    inp.temperature = np.repeat(inp.temperature, B)
    inp.B = B
    return inp


def target_logits(inp, seed=9, scale=1.5):
    rng = np.random.default_rng(seed)
    t = (rng.standard_normal((inp.gamma + 1, inp.V)) * scale).astype(np.float32)
    return np.ascontiguousarray(np.broadcast_to(t, (inp.B, inp.gamma + 1, inp.V))), t.astype(np.float64)


def draft_probs_first(inp):
    """p_d at position 1 of the (identical) blocks: softmax(U_1 + W1[x0] W2)."""
    z = inp.U[0, 0].astype(np.float64) + inp.W1[inp.anchor[0]].astype(np.float64) @ inp.W2.astype(np.float64)
    return softmax(z)


def run(inp, tgt, tau=-1.0, seed=3, offset=0):
    d = oracle.draft_block(inp, seed=seed, offset=offset)
    v = oracle.verify_block(inp, d["tokens"], d["logp"], d["surv"], tgt, tau, seed=seed, offset=offset)
    return d, v


def chi2_p(samples, p, V):
    counts = np.bincount(samples, minlength=V).astype(np.float64)
    exp = p * counts.sum()
    keep = exp > 0
    return stats.chisquare(counts[keep], exp[keep] * counts[keep].sum() / exp[keep].sum()).pvalue


def test_emitted_tokens_follow_the_target():
    inp = tiny()
    tgt, t = target_logits(inp)
    d, v = run(inp, tgt)
    first = np.where(v["accept"] >= 1, d["tokens"][:, 0], v["next"])
    assert chi2_p(first, softmax(t[0]), inp.V) > 1e-3
    # power: the drafter's own first token is far from the target here
    assert chi2_p(d["tokens"][:, 0], softmax(t[0]), inp.V) < 1e-6
    sel = v["accept"] >= 1
    second = np.where(v["accept"][sel] >= 2, d["tokens"][sel, 1], v["next"][sel])
    assert chi2_p(second, softmax(t[1]), inp.V) > 1e-3
    # after two acceptances the bonus token follows position 3 of the target
    full = v["accept"] == 2
    assert full.sum() > 500
    assert chi2_p(v["next"][full], softmax(t[2]), inp.V) > 1e-3


def test_acceptance_rate_is_one_minus_tv():
    inp = tiny(B=40000, seed=6)
    tgt, t = target_logits(inp, seed=10)
    d, v = run(inp, tgt, seed=4)
    c_star = np.minimum(draft_probs_first(inp), softmax(t[0])).sum()
    rate = (v["accept"] >= 1).mean()
    se = np.sqrt(c_star * (1 - c_star) / inp.B)
    assert abs(rate - c_star) < 5 * se, (rate, c_star)
    # the reported acceptance probability is min(1, p_t/p_d) of the drafted token
    pd = np.exp(d["logp"][:, 0])
    pt = softmax(t[0])[d["tokens"][:, 0]]
    assert np.allclose(v["accept_prob"][:, 0], np.minimum(1.0, pt / pd), rtol=1e-9)


def test_trimming_everything_still_emits_from_the_target():
    inp = tiny(B=20000, seed=7)
    tgt, t = target_logits(inp, seed=11)
    d, v = run(inp, tgt, tau=2.0)
    assert (v["keep"] == 0).all() and (v["accept"] == 0).all()
    assert chi2_p(v["next"], softmax(t[0]), inp.V) > 1e-3


def test_trim_counts_the_leading_survivals():
    inp = tiny(B=3, gamma=3, seed=8)
    tgt, _ = target_logits(inp, seed=12)
    d = oracle.draft_block(inp, seed=1)
    surv = np.array([[0.9, 0.5, 0.2], [0.3, 0.2, 0.1], [1.0, 0.99, 0.98]])
    v = oracle.verify_block(inp, d["tokens"], d["logp"], surv, tgt, 0.4, seed=1)
    assert list(v["keep"]) == [2, 0, 3]
    assert (v["accept"] <= v["keep"]).all()
    assert np.isnan(v["accept_prob"][0, 2]) and np.isnan(v["accept_prob"][1]).all()


def test_greedy_verification():
    inp = tiny(B=1, V=6, gamma=3, seed=13, temperature=0.0)
    t = np.zeros((1, 4, 6), np.float32)
    t[0, 0, 2] = 5.0   # target argmax 2, 4, 1, 3 at the four positions
    t[0, 1, 4] = 5.0
    t[0, 2, 1] = 5.0
    t[0, 3, 3] = 5.0
    logp = np.zeros((1, 3))
    surv = np.ones((1, 3))
    v = oracle.verify_block(inp, np.array([[2, 4, 5]]), logp, surv, t, 0.0)
    assert (v["keep"][0], v["accept"][0], v["next"][0]) == (3, 2, 1)
    v = oracle.verify_block(inp, np.array([[2, 4, 1]]), logp, surv, t, 0.0)
    assert (v["accept"][0], v["next"][0]) == (3, 3)
    v = oracle.verify_block(inp, np.array([[0, 4, 1]]), logp, surv, t, 0.0)
    assert (v["accept"][0], v["next"][0]) == (0, 2)


def test_target_equal_to_the_drafter_accepts_everything():
    inp = tiny(B=2000, V=7, gamma=1, seed=14)
    z = inp.U[0, 0].astype(np.float64) + inp.W1[inp.anchor[0]].astype(np.float64) @ inp.W2.astype(np.float64)
    t = np.zeros((inp.B, 2, inp.V), np.float32)
    t[:, 0] = z.astype(np.float32)
    t[:, 1] = 1.0
    d = oracle.draft_block(inp, seed=2)
    v = oracle.verify_block(inp, d["tokens"], d["logp"], d["surv"], t, -1.0, seed=2)
    # p_t = p_d up to float32 rounding of the target logits: acceptance is
    # certain unless u falls within that rounding of 1
    assert (v["accept"] == 1).mean() > 0.999


def test_out_of_range_token_is_rejected():
    inp = tiny(B=2)
    tgt, _ = target_logits(inp)
    with pytest.raises(ValueError):
        oracle.verify_block(inp, np.array([[0, 1], [inp.V, 0]]), np.zeros((2, 2)), np.ones((2, 2)), tgt, 0.0)
