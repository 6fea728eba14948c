"""Pins for the oracle's teacher-forced loss path (CPU only).

Eq 8-12 as transcribed on the dormouse verification page, section 1; the
closed forms for c* come from the Meridian note (Prop 1) and the dormouse
delta table (D7: one-hot against uniform gives 1/V).  Gradients are pinned
by central finite differences and invariants, not by restating the formula.
"""
import math
import os

import numpy as np
import pytest
from scipy import special

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def train_inputs(V=8, r=4, d=5, gamma=3, N=2, dtype="f32", seed=5, **kw):
    base = dict(u_std=1.0, h_std=1.0, w1_std=0.5, w2_std=0.5, wconf_std=0.3,
                anchors="uniform", target_noise_std=1.0)
    base.update(kw)
    return synth.make_inputs(V=V, r=r, d=d, gamma=gamma, B=N, dtype=dtype, seed=seed, **base)


def f64(inp, a):
    return inp.as_f32(a).astype(np.float64)


def prev_tokens(inp):
    return np.concatenate([inp.anchor[:, None], inp.labels[:, :-1]], axis=1)


# --------------------------------------------------------- position weights

def test_position_weights_printed_values(oracle_lib):
    # dormouse page, delta-table row D2 prints w for gamma = 4 and gamma = 7.
    rows = {}
    with open(os.path.join(GOLDEN, "position_weights.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                g, *vals = line.split()
                rows[int(g)] = [float(v) for v in vals]
    w4 = oracle_lib.position_weights(4)
    assert np.array_equal(np.round(w4, 2), rows[4])
    # gamma = 7: the printed list rounds the closed form except at k = 5 and
    # k = 7, where it is 0.01 high (0.5647 and 0.4244); the closed form governs.
    w7 = oracle_lib.position_weights(7)
    assert np.all(np.abs(w7 - rows[7]) <= 0.0101)
    assert np.sum(np.round(w7, 2) != rows[7]) == 2


def test_position_weights_closed_form(oracle_lib):
    w = oracle_lib.position_weights(7)
    assert w[0] == 1.0
    assert abs(w.sum() - (1 - math.exp(-1)) / (1 - math.exp(-1 / 7))) < 1e-14
    assert np.all(np.diff(w) < 0)


# --------------------------------------------------------------------- c*

def _one_row(oracle_lib, U_row, T_row, label=0, w2_zero=True):
    V = len(U_row)
    inp = train_inputs(V=V, gamma=1, N=1)
    inp.U = np.asarray(U_row, np.float32).reshape(1, 1, V)
    inp.target = np.asarray(T_row, np.float32).reshape(1, 1, V)
    inp.labels = np.array([[label]], np.int32)
    if w2_zero:
        inp.W2 = np.zeros_like(inp.W2)
    return oracle_lib.block_loss(inp)


def test_c_star_is_one_for_equal_distributions(oracle_lib):
    rng = np.random.default_rng(0)
    # multiples of 2^-10 below 8 in magnitude, so U + 4 is exact in float32
    U = (np.round(rng.standard_normal(37) * 1024) / 1024).astype(np.float32)
    out = _one_row(oracle_lib, U, U)
    assert out["c_star"][0] == 1.0 and out["tv"][0] == 0.0
    # softmax is shift invariant: the same distribution from shifted logits
    out = _one_row(oracle_lib, U, U + np.float32(4.0))
    assert abs(out["c_star"][0] - 1.0) < 1e-13


def test_c_star_one_hot_against_uniform_is_one_over_V(oracle_lib):
    for V in (2, 5, 64):
        T = np.zeros(V, np.float32)
        T[1] = 2000.0  # exp(-2000) underflows: an exact one-hot target
        out = _one_row(oracle_lib, np.zeros(V, np.float32), T)
        assert abs(out["c_star"][0] - 1.0 / V) < 1e-15


def test_c_star_point_mass_drafter_equals_target_mass(oracle_lib):
    # Meridian note, Prop 1: for p_d = delta at x, c* = p_t(x).
    rng = np.random.default_rng(1)
    V = 23
    T = rng.standard_normal(V).astype(np.float32)
    for x in (0, 7, 22):
        U = np.zeros(V, np.float32)
        U[x] = 2000.0
        out = _one_row(oracle_lib, U, T)
        pt = special.softmax(T.astype(np.float64))
        assert abs(out["c_star"][0] - pt[x]) < 1e-14


def test_c_star_disjoint_supports_is_zero(oracle_lib):
    U = np.zeros(6, np.float32); U[1] = 2000.0
    T = np.zeros(6, np.float32); T[4] = 2000.0
    out = _one_row(oracle_lib, U, T)
    assert out["c_star"][0] == 0.0 and out["tv"][0] == 2.0


def test_bounds_on_random_rows(oracle_lib):
    inp = train_inputs(V=50, N=6, gamma=4, u_std=3.0)
    out = oracle_lib.block_loss(inp)
    assert np.all((out["c_star"] >= 0) & (out["c_star"] <= 1))
    assert np.all((out["tv"] >= 0) & (out["tv"] <= 2))
    assert np.all(out["ce"] >= 0)
    # Gibbs: the cross-entropy against c is at least the entropy of c*
    cs = out["c_star"]
    hb = -(special.xlogy(cs, cs) + special.xlogy(1 - cs, 1 - cs))
    assert np.all(out["bce"] >= hb - 1e-12)
    # the confidence gradient pushes c toward c*
    assert np.all(np.sign(out["dA"]) == np.sign(out["conf"] - cs))


# ---------------------------------------------------------- reductions

def test_cross_entropy_only_reduces_to_textbook(oracle_lib):
    # alpha = (1, 0, 0): L = mean over blocks of sum_k w_k (-log softmax(z_d)[x*]),
    # with the library log-softmax; dZ = (w_k / N)(softmax(z_d) - onehot).
    inp = train_inputs(V=30, N=4, gamma=5)
    out = oracle_lib.block_loss(inp, alpha=(1.0, 0.0, 0.0))
    U, W1, W2 = f64(inp, inp.U), f64(inp, inp.W1), f64(inp, inp.W2)
    zd = U + W1[prev_tokens(inp)] @ W2
    ls = special.log_softmax(zd, axis=-1)
    w = oracle_lib.position_weights(inp.gamma)
    nll = -np.take_along_axis(ls, inp.labels[..., None], axis=-1)[..., 0]
    assert abs(out["loss4"][0] - (nll * w).sum() / inp.B) < 1e-12
    onehot = np.eye(inp.V)[inp.labels]
    want = (w[None, :, None] / inp.B) * (np.exp(ls) - onehot)
    assert np.allclose(out["dZ"].reshape(want.shape), want, atol=1e-15)


def test_loss_combination_and_terms(oracle_lib):
    inp = train_inputs(V=30, N=3, gamma=4)
    out = oracle_lib.block_loss(inp, alpha=(0.1, 0.9, 1.0))
    L, Lce, Ltv, Lconf = out["loss4"]
    assert abs(L - (0.1 * Lce + 0.9 * Ltv + 1.0 * Lconf)) < 1e-14
    w = np.tile(oracle_lib.position_weights(inp.gamma), inp.B)
    assert abs(Ltv - (w * 2 * (1 - out["c_star"])).sum() / inp.B) < 1e-12


def test_dz_rows_sum_to_zero(oracle_lib):
    inp = train_inputs(V=40, N=3, gamma=4, u_std=2.0)
    out = oracle_lib.block_loss(inp)
    assert np.all(np.abs(out["dZ"].sum(axis=1)) < 1e-15)


# ---------------------------------------------------------- finite differences

def _perturbed(inp, field, idx, delta):
    a = getattr(inp, field).copy()
    a[idx] = np.float32(a[idx] + delta)
    step = float(a[idx]) - float(getattr(inp, field)[idx])
    c = synth.Inputs(**{f: getattr(inp, f) for f in inp.__dataclass_fields__})
    setattr(c, field, a)
    return c, step


def _fd(oracle_lib, inp, field, idx, alpha, h=1e-3):
    plus, sp = _perturbed(inp, field, idx, h)
    minus, sm = _perturbed(inp, field, idx, -h)
    lp = oracle_lib.block_loss(plus, alpha=alpha, want_dZ=False, want_dW2=False)["loss4"][0]
    lm = oracle_lib.block_loss(minus, alpha=alpha, want_dZ=False, want_dW2=False)["loss4"][0]
    return (lp - lm) / (sp - sm)


def _away_from_kinks(oracle_lib, inp):
    """Finite differences are valid only away from |p_d - p_t| = 0."""
    U, W1, W2, T = f64(inp, inp.U), f64(inp, inp.W1), f64(inp, inp.W2), f64(inp, inp.target)
    zd = U + W1[prev_tokens(inp)] @ W2
    gap = np.abs(special.softmax(zd, -1) - special.softmax(T, -1))
    return gap.min() > 2e-3


@pytest.mark.parametrize("alpha", [(0.1, 0.9, 0.0), (0.0, 1.0, 0.0), (1.0, 0.0, 0.0)])
def test_dz_matches_finite_differences(oracle_lib, alpha):
    # c* is a label (stop-gradient), so the confidence term is excluded here.
    inp = train_inputs(V=8, r=4, N=2, gamma=3, seed=21)
    assert _away_from_kinks(oracle_lib, inp)
    out = oracle_lib.block_loss(inp, alpha=alpha)
    dZ = out["dZ"].reshape(inp.B, inp.gamma, inp.V)
    for idx in [(0, 0, 0), (0, 1, 3), (1, 2, 7), (1, 0, 5), (0, 2, 2)]:
        fd = _fd(oracle_lib, inp, "U", idx, alpha)
        assert abs(fd - dZ[idx]) < 1e-6 + 1e-5 * abs(dZ[idx]), (idx, fd, dZ[idx])


def test_dw2_matches_finite_differences(oracle_lib):
    alpha = (0.1, 0.9, 0.0)
    inp = train_inputs(V=8, r=4, N=2, gamma=3, seed=21)
    assert _away_from_kinks(oracle_lib, inp)
    out = oracle_lib.block_loss(inp, alpha=alpha)
    for idx in [(0, 0), (1, 3), (3, 7), (2, 5)]:
        fd = _fd(oracle_lib, inp, "W2", idx, alpha)
        assert abs(fd - out["dW2"][idx]) < 1e-6 + 1e-5 * abs(out["dW2"][idx]), idx


def test_da_matches_finite_differences_in_confidence_weights(oracle_lib):
    # dL/dw_m = sum_i dA_i [h_i; e_i]_m, and c* does not depend on w.
    alpha = (0.1, 0.9, 1.0)
    inp = train_inputs(V=8, r=4, d=5, N=2, gamma=3, seed=21)
    out = oracle_lib.block_loss(inp, alpha=alpha)
    h = f64(inp, inp.h).reshape(-1, inp.d)
    e = f64(inp, inp.W1)[prev_tokens(inp).reshape(-1)]
    grad_w = out["dA"] @ np.concatenate([h, e], axis=1)
    for m in (0, 3, inp.d, inp.d + 3):
        fd = _fd(oracle_lib, inp, "w_conf", (m,), alpha)
        assert abs(fd - grad_w[m]) < 1e-7 + 1e-5 * abs(grad_w[m]), m


# ---------------------------------------------------------- wiring

def test_off_by_one_gate_training(oracle_lib):
    # dormouse page, section 7 item 1: position k is fed x_{k-1} (the anchor
    # at k = 1) and its CE target is x_k.  W1 row v encodes v; the confidence
    # weights read only that column, so c reveals the token that was fed.
    inp = train_inputs(V=64, r=2, d=3, N=3, gamma=5)
    W1 = np.zeros((64, 2), np.float32); W1[:, 0] = np.arange(64) / 128.0
    w = np.zeros(5, np.float32); w[3] = 1.0
    inp.W1, inp.w_conf = W1, w
    inp.labels = np.arange(15, dtype=np.int32).reshape(3, 5) + 10
    out = oracle_lib.block_loss(inp)
    fed = np.rint(special.logit(out["conf"]) * 128).astype(int).reshape(3, 5)
    assert np.array_equal(fed, prev_tokens(inp))
    # CE target is the label at the same position: with W2 = 0, ce = -log_softmax(U)[x_k]
    inp.W2 = np.zeros_like(inp.W2)
    out = oracle_lib.block_loss(inp)
    ls = special.log_softmax(f64(inp, inp.U), -1)
    want = -np.take_along_axis(ls, inp.labels[..., None], -1)[..., 0].reshape(-1)
    assert np.allclose(out["ce"], want, atol=1e-12)


def test_teacher_forced_path_equals_sampled_path(oracle_lib):
    # Feeding the sampled tokens back as labels reproduces the sampler's
    # conditioning: same confidence, and ce = -logp at T = 1.
    inp = train_inputs(V=50, r=4, d=6, N=4, gamma=5, u_std=2.0)
    inp.temperature = np.ones(inp.B, np.float32)
    smp = oracle_lib.draft_block(inp, seed=17)
    inp.labels = smp["tokens"].astype(np.int32)
    out = oracle_lib.block_loss(inp)
    assert np.allclose(out["conf"], smp["conf"].reshape(-1), atol=1e-15)
    assert np.allclose(out["ce"], -smp["logp"].reshape(-1), atol=1e-12)


def test_row_subset_matches_full(oracle_lib):
    inp = train_inputs(V=30, N=3, gamma=4)
    full = oracle_lib.block_loss(inp)
    rows = np.array([0, 5, 11, 7])
    sub = oracle_lib.block_loss(inp, rows=rows, want_dW2=False)
    for key in ("c_star", "conf", "dA", "ce", "tv", "bce"):
        assert np.array_equal(sub[key], full[key][rows])
    assert np.array_equal(sub["dZ"], full["dZ"][rows])


def test_dw2_equals_embedding_transpose_times_dz(oracle_lib):
    inp = train_inputs(V=30, r=5, N=3, gamma=4)
    out = oracle_lib.block_loss(inp)
    E = f64(inp, inp.W1)[prev_tokens(inp).reshape(-1)]
    assert np.allclose(out["dW2"], E.T @ out["dZ"], atol=1e-15)


def test_rejects_out_of_range_label(oracle_lib):
    inp = train_inputs(V=10)
    inp.labels = inp.labels.copy()
    inp.labels[0, 1] = 10
    with pytest.raises(ValueError):
        oracle_lib.block_loss(inp)


# --------------------------------------------------------- rest of the backward
# dW1, dw and dh from the loss's own dZ and dA, each against central finite
# differences of the oracle's loss.  c* is a label (held constant), so each
# check picks inputs where c* does not move with the perturbed parameter:
# alpha_conf = 0 for the path through z_d, W2 = 0 (z_d independent of W1)
# for the confidence path of dW1, and h (which never enters z_d).

def _backward(oracle_lib, inp, alpha):
    out = oracle_lib.block_loss(inp, alpha=alpha)
    return oracle_lib.block_loss_backward(inp, out["dZ"], out["dA"])


def test_dw1_through_the_bias_matches_finite_differences(oracle_lib):
    alpha = (0.1, 0.9, 0.0)
    inp = train_inputs(V=8, r=4, N=2, gamma=3, seed=21)
    assert _away_from_kinks(oracle_lib, inp)
    g = _backward(oracle_lib, inp, alpha)["dW1"]
    fed = sorted(set(prev_tokens(inp).reshape(-1).tolist()))
    for x in fed[:3]:
        for j in (0, 3):
            fd = _fd(oracle_lib, inp, "W1", (x, j), alpha)
            assert abs(fd - g[x, j]) < 1e-6 + 1e-5 * abs(g[x, j]), (x, j, fd, g[x, j])


def test_dw1_through_the_confidence_matches_finite_differences(oracle_lib):
    alpha = (0.1, 0.9, 1.0)
    inp = train_inputs(V=8, r=4, N=2, gamma=3, seed=22, w2_std=0.0)
    assert not np.any(inp.W2)
    g = _backward(oracle_lib, inp, alpha)["dW1"]
    fed = sorted(set(prev_tokens(inp).reshape(-1).tolist()))
    for x in fed[:3]:
        for j in (1, 2):
            fd = _fd(oracle_lib, inp, "W1", (x, j), alpha)
            assert abs(fd - g[x, j]) < 1e-7 + 1e-5 * abs(g[x, j]), (x, j, fd, g[x, j])


def test_dw1_rows_of_tokens_never_fed_are_zero(oracle_lib):
    inp = train_inputs(V=16, r=4, N=2, gamma=3, seed=23)
    g = _backward(oracle_lib, inp, (0.1, 0.9, 1.0))["dW1"]
    fed = set(prev_tokens(inp).reshape(-1).tolist())
    for x in range(inp.V):
        if x not in fed:
            assert not np.any(g[x])
        else:
            assert np.any(g[x])


def test_dh_matches_finite_differences(oracle_lib):
    alpha = (0.1, 0.9, 1.0)
    inp = train_inputs(V=8, r=4, d=5, N=2, gamma=3, seed=24)
    dh = _backward(oracle_lib, inp, alpha)["dh"].reshape(inp.B, inp.gamma, inp.d)
    for idx in [(0, 0, 0), (1, 2, 4), (0, 1, 2)]:
        fd = _fd(oracle_lib, inp, "h", idx, alpha)
        assert abs(fd - dh[idx]) < 1e-7 + 1e-5 * abs(dh[idx]), (idx, fd, dh[idx])


def test_dw_conf_matches_finite_differences(oracle_lib):
    alpha = (0.1, 0.9, 1.0)
    inp = train_inputs(V=8, r=4, d=5, N=2, gamma=3, seed=25)
    dw = _backward(oracle_lib, inp, alpha)["dw"]
    for m in (0, 2, inp.d, inp.d + 3):
        fd = _fd(oracle_lib, inp, "w_conf", (m,), alpha)
        assert abs(fd - dw[m]) < 1e-7 + 1e-5 * abs(dw[m]), (m, fd, dw[m])


def test_column_subset_returns_the_same_values(oracle_lib):
    oracle = oracle_lib
    # the column-subset outputs are the full outputs at those columns (the
    # full-size GPU check relies on this to avoid R x V float64 values)
    inp = synth.make_inputs(V=300, r=16, d=8, gamma=3, B=4, dtype="bf16", seed=71, w1_std=0.3,
                            w2_std=0.3, anchors="uniform", target_noise_std=1.0)
    full = oracle.block_loss(inp)
    cols = np.array([299, 0, 17, 150, 17])
    sub = oracle.block_loss(inp, cols=cols)
    assert np.array_equal(sub["dZ"], full["dZ"][:, cols])
    assert np.allclose(sub["dW2"], full["dW2"][:, cols], rtol=1e-12, atol=1e-15)
    for k in ("loss4", "c_star", "conf", "dA"):
        assert np.array_equal(sub[k], full[k]), k
    rows = np.array([5, 0, 11])
    part = oracle.block_loss(inp, rows=rows, cols=cols, want_dW2=False)
    assert np.array_equal(part["dZ"], full["dZ"][rows][:, cols])
