"""GPU parity of dspark_block_loss_backward against the CPU oracle (through
the C ABI).

The backward call takes the loss call's own dZ and dA (as the GPU stored
them); the oracle is given the very same values, widened to float64, so the
comparison isolates the backward arithmetic.

Tolerances are worst-case rounding bounds of the GPU's float32 sums, from
the absolute-value sums A of the terms (float64 here):
  dE_ij   the matrix cores add 32 exact bf16 x bf16 products per step and
          accumulate in float32, ceil(V / 32) steps, then the vocabulary
          slices and the dA w term: (V/32 + S + 2) 2^-24 A_ij; float32 dZ
          enters as hi + lo bf16, exact to 2^-18 of itself: + 2^-18 A_ij.
  dW1     the dE rows of a token added in row order: the sum of the rows'
          bounds plus (rows + 2) 2^-24 of the sum of their A.
  dw_conf fused multiply-adds in row order within 64 row splits, then the
          splits: (R/64 + 64 + 2) 2^-24 sum |dA x|.
  dh      one product: 2^-23 |dA w|.
"""
import numpy as np
import pytest

import oracle
import synth
from _parity import note, rel_l2

pytestmark = pytest.mark.gpu

U24 = 2.0 ** -24


@pytest.fixture(scope="module")
def ops():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from semi_autoregressive_draft_markov_amd import binding, ops as _ops
    binding.load()
    return _ops


def small(**kw):
    base = dict(V=1000, r=64, d=48, gamma=5, B=6, dtype="bf16", head="markov", seed=31,
                u_std=3.0, h_std=1.0, w1_std=0.25, w2_std=0.25, wconf_std=0.1,
                anchors="uniform", target_noise_std=1.5)
    base.update(kw)
    return synth.make_inputs(**base)


def prev_tokens(inp):
    return np.concatenate([inp.anchor[:, None], inp.labels[:, :-1]], axis=1).reshape(-1)


def run_gpu(ops, inp, dl="bf16", want=(True, True, True), t=None):
    """Loss call then backward call on the GPU; numpy copies of dZ, dA and
    the three gradients."""
    import torch
    if t is None:
        t = synth.to_torch(inp)
    lo = ops.block_loss(t["U"], t["target"], t["h"], t["anchor"], t["labels"], t["W1"], t["W2"],
                        t["w_conf"], dlogits_dtype=dl, want_dW2=False)
    bo = ops.block_loss_backward(lo["dlogits"], lo["dconf_logit"], t["h"], t["anchor"],
                                 t["labels"], t["W1"], t["W2"], t["w_conf"], want_dW1=want[0],
                                 want_dw_conf=want[1], want_dh=want[2])
    torch.cuda.synchronize()
    res = dict(dA=lo["dconf_logit"].cpu().numpy().reshape(-1), _lo=lo, _bo=bo)
    res["dZ"] = lo["dlogits"].float().cpu().numpy().reshape(inp.B * inp.gamma, inp.V)
    for k in ("dW1", "dw_conf", "dh"):
        res[k] = None if bo[k] is None else bo[k].cpu().numpy()
    return res


def bounds(inp, dZ, dA, f32z: bool, slices: int):
    """Per-entry error bounds of dE, dW1, dw_conf and dh (see the module doc)."""
    R, V, r, d = inp.B * inp.gamma, inp.V, inp.r, inp.d
    W2 = np.abs(inp.as_f32(inp.W2).astype(np.float64))
    w = inp.as_f32(inp.w_conf).astype(np.float64)
    prev = prev_tokens(inp)
    valid = (prev >= 0) & (prev < V) & np.isfinite(dA)
    dAv = np.where(valid, dA, 0.0)
    A = np.abs(np.nan_to_num(dZ)) @ W2.T + np.abs(dAv)[:, None] * np.abs(w[d:])[None, :]
    steps = -(-V // 32)
    tol_de = (steps + slices + 2) * U24 * A + (2.0 ** -18 * A if f32z else 0.0)
    tol_w1 = np.zeros((V, r))
    a_w1 = np.zeros((V, r))
    cnt = np.zeros(V)
    for i in np.nonzero(valid)[0]:
        tol_w1[prev[i]] += tol_de[i]
        a_w1[prev[i]] += A[i]
        cnt[prev[i]] += 1
    tol_w1 += (cnt + 2)[:, None] * U24 * a_w1
    h = np.abs(inp.as_f32(inp.h).astype(np.float64).reshape(R, d))
    E = np.abs(inp.as_f32(inp.W1).astype(np.float64)[np.where(valid, prev, 0)])
    X = np.concatenate([h, E], axis=1)
    tol_dw = (R / 64 + 64 + 2) * U24 * (np.abs(dAv) @ X)
    tol_dh = 2.0 * U24 * np.abs(dA)[:, None] * np.abs(w[:d])[None, :]
    return tol_w1, tol_dw, tol_dh


def check(inp, g, label, f32z, slices=256):
    ref = oracle.block_loss_backward(inp, g["dZ"], g["dA"])
    tol_w1, tol_dw, tol_dh = bounds(inp, g["dZ"], g["dA"], f32z, slices)
    err = np.abs(g["dW1"] - ref["dW1"])
    assert (err <= tol_w1 + 1e-30).all(), \
        "%s: dW1 max err/bound %.3g" % (label, (err / np.maximum(tol_w1, 1e-30)).max())
    assert rel_l2(g["dW1"], ref["dW1"]) <= 1e-5, label
    err = np.abs(g["dw_conf"] - ref["dw"])
    assert (err <= tol_dw + 1e-30).all(), \
        "%s: dw_conf max err/bound %.3g" % (label, (err / np.maximum(tol_dw, 1e-30)).max())
    dh = g["dh"].reshape(ref["dh"].shape)
    fin = np.isfinite(ref["dh"])
    assert (np.abs(dh - ref["dh"])[fin] <= tol_dh[fin]).all(), label
    assert np.array_equal(np.isnan(dh), np.isnan(ref["dh"])), label
    # tokens never fed get exact zeros
    fed = np.zeros(inp.V, bool)
    prev = prev_tokens(inp)
    fed[prev[(prev >= 0) & (prev < inp.V)]] = True
    assert not g["dW1"][~fed].any(), label


@pytest.mark.parametrize("dl", ["bf16", "f32"])
def test_matrix_core_ragged(ops, dl):
    # V = 1000 (ragged last stage), R = 30 rows (one partial 256-row tile)
    inp = small()
    note("case: bwd mfma V1000 r64 N6 dlogits %s" % dl)
    check(inp, run_gpu(ops, inp, dl), "ragged " + dl, dl == "f32")


@pytest.mark.parametrize("dl", ["bf16", "f32"])
def test_rank256_two_tiles(ops, dl):
    # R = 280 rows: two row tiles, the second ragged; many vocabulary slices
    inp = small(V=4104, r=256, d=64, gamma=7, B=40, seed=32)
    note("case: bwd mfma V4104 r256 N40 dlogits %s" % dl)
    check(inp, run_gpu(ops, inp, dl), "r256 " + dl, dl == "f32")


@pytest.mark.parametrize("r", [32, 96, 160, 224])
def test_other_matrix_core_ranks(ops, r):
    inp = small(V=520, r=r, d=40, gamma=4, B=5, seed=33 + r)
    note("case: bwd mfma V520 r%d" % r)
    check(inp, run_gpu(ops, inp, "bf16"), "r%d" % r, False)


def test_vector_path(ops):
    inp = small(V=999, r=48, d=20, gamma=3, B=4, seed=34)
    note("case: bwd vector V999 r48")
    check(inp, run_gpu(ops, inp, "f32"), "vector", False)


def test_fp32_tiny(ops):
    inp = synth.config_inputs(1)
    note("case: bwd fp32 V1024 r32 N4")
    check(inp, run_gpu(ops, inp, "f32"), "fp32 tiny", False)


def test_one_token_fed_to_every_row(ops):
    # 210 rows all fed token 5: one sorted segment of four 64-row chunks
    inp = small(V=1000, r=64, d=32, gamma=7, B=30, seed=35)
    inp.anchor = np.full_like(inp.anchor, 5)
    inp.labels = np.full_like(inp.labels, 5)
    note("case: bwd one token, 210 rows")
    g = run_gpu(ops, inp, "bf16")
    check(inp, g, "one token", False)
    assert np.count_nonzero(np.abs(g["dW1"]).sum(axis=1)) == 1


def test_bad_token_rows_are_left_out(ops):
    from semi_autoregressive_draft_markov_amd import binding
    inp = small(seed=36)
    inp.labels = inp.labels.copy()
    # block 2: the loss gives NaN dA at the rows that predict (k = 1) and are
    # fed (k = 2) the bad label; the backward also finds prev out of range
    inp.labels[2, 1] = inp.V
    note("case: bwd out-of-range label")
    g = run_gpu(ops, inp, "bf16")
    dA2 = g["dA"].reshape(inp.B, inp.gamma)[2]
    assert np.isnan(dA2[1:3]).all() and np.isfinite(dA2[[0, 3, 4]]).all()
    bo = g["_bo"]
    assert binding.dspark_read_device_error(bo["_dims"], bo["_ws"]) == 1
    assert np.isfinite(g["dW1"]).all() and np.isfinite(g["dw_conf"]).all()
    check(inp, g, "bad token", False)


def test_optional_outputs_and_determinism(ops):
    inp = small(seed=37)
    a = run_gpu(ops, inp, "bf16")
    b = run_gpu(ops, inp, "bf16")
    for k in ("dW1", "dw_conf", "dh"):
        assert np.array_equal(a[k], b[k]), k
    c = run_gpu(ops, inp, "bf16", want=(True, False, False))
    assert np.array_equal(a["dW1"], c["dW1"]) and c["dw_conf"] is None and c["dh"] is None
    e = run_gpu(ops, inp, "bf16", want=(False, True, True))
    assert np.array_equal(a["dw_conf"], e["dw_conf"]) and np.array_equal(a["dh"], e["dh"])


def rows_as_blocks(inp, rows):
    """The listed teacher-forced rows as a problem of their own: one block of
    length 1 per row, whose anchor is the token that row was fed and whose
    hidden state is that row's.  Every per-row term of the backward (dE_i,
    its scatter into dW1, dA_i [h_i; e_i], dA_i w) depends on the row only
    through these, so the oracle's sums over this problem are its sums over
    the listed rows of the original one."""
    import dataclasses
    prev = prev_tokens(inp)
    R = inp.B * inp.gamma
    return dataclasses.replace(
        inp, B=len(rows), gamma=1, anchor=np.ascontiguousarray(prev[rows].astype(np.int32)),
        labels=np.zeros((len(rows), 1), np.int32), h=np.ascontiguousarray(inp.h.reshape(R, 1, inp.d)[rows]),
        U=None, target=None, temperature=np.ones(len(rows), np.float32))


def test_qwen3_8b_shape_against_the_oracle(ops):
    """7168 rows, V = 151936, r = 256, d = 4096, from the GPU's own dZ and
    dA (both dlogits dtypes): dW1 in full on the rows of tokens of every
    frequency class (all rows fed those tokens, through the oracle), and
    dw_conf and dh over all rows against the oracle."""
    import torch
    inp = synth.config_inputs(3)
    R, V, r, d = inp.B * inp.gamma, inp.V, inp.r, inp.d
    note("case: bwd qwen3-8b-shaped V151936 r256 N1024 (7168 rows)")
    t = synth.to_torch(inp)
    prev = prev_tokens(inp)
    uniq, counts = np.unique(prev, return_counts=True)
    order = np.argsort(-counts, kind="stable")
    toks = np.concatenate([uniq[order[:3]], uniq[order[len(order) // 2:len(order) // 2 + 2]],
                           uniq[order[-2:]]])
    rows = np.nonzero(np.isin(prev, toks))[0]
    sub = rows_as_blocks(inp, rows)
    W2 = np.abs(inp.as_f32(inp.W2).astype(np.float64))
    w = inp.as_f32(inp.w_conf).astype(np.float64)
    hq = np.abs(inp.as_f32(inp.h).reshape(R, d).astype(np.float64))
    E = np.abs(inp.as_f32(inp.W1).astype(np.float64)[prev])
    for dl in ("bf16", "f32"):
        note("  dlogits %s (%d rows feed the %d sampled tokens)" % (dl, len(rows), len(toks)))
        lo = ops.block_loss(t["U"], t["target"], t["h"], t["anchor"], t["labels"], t["W1"],
                            t["W2"], t["w_conf"], dlogits_dtype=dl, want_dW2=False)
        bo = ops.block_loss_backward(lo["dlogits"], lo["dconf_logit"], t["h"], t["anchor"],
                                     t["labels"], t["W1"], t["W2"], t["w_conf"])
        torch.cuda.synchronize()
        dA = lo["dconf_logit"].cpu().numpy().reshape(-1).astype(np.float64)
        dz = lo["dlogits"].view(R, V)
        Z = dz[torch.as_tensor(rows, device=dz.device)].double().cpu().numpy()
        ref = oracle.block_loss_backward(sub, Z, dA[rows], want_dw=False, want_dh=False)
        dW1 = bo["dW1"].cpu().numpy()
        # tolerance per token: the float32 bound of the module docstring
        # from the absolute-value sums of that token's rows
        A_rows = np.abs(Z) @ W2.T + np.abs(dA[rows])[:, None] * np.abs(w[d:])[None, :]
        steps = -(-V // 32)
        for x in toks:
            mine = prev[rows] == x
            A = A_rows[mine].sum(axis=0)
            tol = (steps + 256 + int(mine.sum()) + 4) * U24 * A + (2.0 ** -18 * A if dl == "f32" else 0)
            err = np.abs(dW1[x] - ref["dW1"][x])
            assert (err <= tol).all(), (dl, int(x), int(mine.sum()), float((err / tol).max()))
        unfed = np.setdiff1d(np.arange(0, V, 997), uniq)
        assert not dW1[unfed].any()
        # dw_conf and dh over every row (dZ plays no part in them)
        refw = oracle.block_loss_backward(inp, None, dA, want_dW1=False)
        X_abs = np.concatenate([hq, E], axis=1)
        tol = (R / 64 + 66) * U24 * (np.abs(dA) @ X_abs)
        got = bo["dw_conf"].cpu().numpy().astype(np.float64)
        assert (np.abs(got - refw["dw"]) <= tol).all(), dl
        dh = bo["dh"].view(R, d).cpu().numpy().astype(np.float64)
        assert (np.abs(dh - refw["dh"]) <= 2 * U24 * np.abs(refw["dh"])).all(), dl
        del lo, bo, dz
