"""GPU parity of dspark_block_loss against the CPU oracle (through the C ABI).

Small problems are compared on every output.  The Qwen3-8B-shaped workload
(7168 rows) is compared with the oracle on every row: the per-row values and
the four losses, dZ on a set of columns of every row (and whole rows on a
sample), and dW2 on those columns.
"""
import numpy as np
import pytest

import oracle
import synth
from _parity import bf16_round, bf16_ulp, check_loss, note, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from semi_autoregressive_draft_markov_amd import binding, ops as _ops
    binding.load()
    return _ops


def run_gpu(ops, inp, dlogits="f32", alpha=None, pos_weight=None, want_dW2=True):
    import torch
    t = synth.to_torch(inp)
    out = ops.block_loss(t["U"], t["target"], t["h"], t["anchor"], t["labels"], t["W1"], t["W2"],
                         t["w_conf"], alpha=alpha, pos_weight=pos_weight, dlogits_dtype=dlogits,
                         want_dW2=want_dW2)
    torch.cuda.synchronize()
    res = {}
    for k_out, k_res in (("loss4", "loss4"), ("c_star", "c_star"), ("conf", "conf"),
                         ("dconf_logit", "dconf"), ("dW2", "dW2")):
        res[k_res] = None if out[k_out] is None else out[k_out].cpu().numpy()
    res["dlogits"] = None if out["dlogits"] is None else out["dlogits"].float().cpu().numpy()
    res["_out"] = out
    return res


def small(**kw):
    base = dict(V=1000, r=64, d=48, gamma=5, B=6, dtype="bf16", head="markov", seed=21,
                u_std=3.0, h_std=1.0, w1_std=0.25, w2_std=0.25, wconf_std=0.1,
                anchors="uniform", target_noise_std=1.5)
    base.update(kw)
    return synth.make_inputs(**base)


def test_tiny_fp32_loss(ops):
    inp = synth.config_inputs(1)
    note("case: tiny fp32 loss V1024 r32 N4")
    g = run_gpu(ops, inp)
    check_loss(inp, g, oracle.block_loss(inp), label="tiny fp32 loss")


@pytest.mark.parametrize("dl", ["f32", "bf16"])
def test_bf16_matrix_core_ragged(ops, dl):
    # V = 1000 (ragged column groups), R = 30 rows (pads to 32), strong bias
    inp = small()
    note("case: bf16 mfma loss V1000 r64 N6 dlogits %s" % dl)
    g = run_gpu(ops, inp, dlogits=dl)
    check_loss(inp, g, oracle.block_loss(inp), label="bf16 ragged " + dl, dz_bf16=dl == "bf16")


def test_rank256_many_rows(ops):
    inp = small(V=4104, r=256, d=64, gamma=7, B=9, seed=22)
    note("case: bf16 mfma loss V4104 r256 N9")
    g = run_gpu(ops, inp)
    check_loss(inp, g, oracle.block_loss(inp), label="r256")


def test_vector_path_odd_shapes(ops):
    inp = small(V=999, r=48, d=20, gamma=3, B=4, seed=23)
    note("case: bf16 vector loss V999 r48")
    g = run_gpu(ops, inp)
    check_loss(inp, g, oracle.block_loss(inp), label="vector path")


def test_custom_alpha_and_weights(ops):
    inp = small(seed=24)
    alpha = (1.0, 0.0, 0.5)
    pw = [1.0, 0.5, 0.25, 0.125, 0.0625]
    g = run_gpu(ops, inp, alpha=alpha, pos_weight=pw)
    check_loss(inp, g, oracle.block_loss(inp, alpha=alpha, pos_weight=pw), label="custom alpha")


def test_equal_distributions_give_c_star_one(ops):
    # target = the draft logits themselves (W2 = 0): c* = 1, tv = 0
    inp = small(seed=25)
    inp.W2 = np.zeros_like(inp.W2)
    inp.target = inp.U.copy()
    g = run_gpu(ops, inp)
    assert np.allclose(g["c_star"], 1.0, atol=1e-5)
    assert abs(g["loss4"][2]) < 1e-4


def test_dz_rows_sum_to_zero_and_deterministic(ops):
    inp = small(seed=26)
    a = run_gpu(ops, inp)
    b = run_gpu(ops, inp)
    for k in ("loss4", "c_star", "dlogits", "dW2"):
        assert np.array_equal(a[k], b[k]), k
    dz = a["dlogits"].reshape(-1, inp.V)
    scale = np.abs(dz).max()
    assert np.abs(dz.sum(axis=1)).max() <= 1e-4 * scale


def test_out_of_range_label_is_flagged(ops):
    from semi_autoregressive_draft_markov_amd import binding
    inp = small(seed=27)
    inp.labels = inp.labels.copy()
    inp.labels[2, 1] = inp.V
    g = run_gpu(ops, inp)
    out = g["_out"]
    assert binding.dspark_read_device_error(out["_dims"], out["_ws"]) == 1
    assert np.isnan(g["loss4"]).all()
    assert np.isnan(g["c_star"][2, 1:3]).all()


def test_qwen3_8b_shape_all_rows(ops):
    """Every one of the 7168 rows against the oracle: c*, c, dL/da per row,
    the four losses, dZ on 64 columns of every row (and in full on 9 rows),
    and dW2 on those columns (the oracle's own dW2 there)."""
    import torch
    inp = synth.config_inputs(3)
    R, V = inp.B * inp.gamma, inp.V
    rng = np.random.default_rng(5)
    cols = np.unique(np.concatenate([
        [0, 1, 15, 16, 255, 256, 4095, 4096, 75000, 131071, 131072, V - 8, V - 1],
        rng.choice(V, 51, replace=False)]))
    rows = np.array([0, 1, 6, 7, 500, 3333, 5000, 7160, 7167])
    note("case: qwen3-8b-shaped loss V151936 r256 N1024, oracle over all 7168 rows")
    ref = oracle.block_loss(inp, cols=cols)
    ref_rows = oracle.block_loss(inp, rows=rows, want_dW2=False)
    per_row = {k: ref[k] for k in ("loss4", "c_star", "conf", "dA")}
    prev = np.concatenate([inp.anchor[:, None], inp.labels[:, :-1]], axis=1).reshape(-1)
    E = synth.bf16_bits_to_f32(inp.W1[prev]).astype(np.float64)
    t = synth.to_torch(inp)
    cidx = torch.as_tensor(cols, device="cuda")
    for dl in ("f32", "bf16"):
        note("  dlogits %s" % dl)
        out = ops.block_loss(t["U"], t["target"], t["h"], t["anchor"], t["labels"], t["W1"],
                             t["W2"], t["w_conf"], dlogits_dtype=dl)
        torch.cuda.synchronize()
        dz = out["dlogits"].view(R, V)
        g = dict(loss4=out["loss4"].cpu().numpy(), c_star=out["c_star"].cpu().numpy(),
                 conf=out["conf"].cpu().numpy(), dconf=out["dconf_logit"].cpu().numpy())
        check_loss(inp, g, per_row, label="qwen3-8b all rows " + dl)
        sub = dict(g, loss4=None)
        sub["dlogits"] = dz[torch.as_tensor(rows, device="cuda")].float().cpu().numpy()
        check_loss(inp, sub, ref_rows, rows=rows, label="qwen3-8b full rows " + dl,
                   dz_bf16=dl == "bf16")
        # dZ on the sampled columns of every row
        got = dz[:, cidx].double().cpu().numpy()
        want = bf16_round(ref["dZ"]) if dl == "bf16" else ref["dZ"]
        assert rel_l2(got, want) <= 2e-3, (dl, rel_l2(got, want))
        assert rel_l2(got, want, axis=0).max() <= 2e-3, dl
        if dl == "bf16":
            # element by element within one bf16 ulp, except where p_d and
            # p_t are so close that sign(p_d - p_t) of the TV subgradient
            # comes out the other way under rounding: such an element moves
            # by 2 alpha_tv w_k p_d / N (sign at equality is a reading; the
            # norm-wise bounds above cover these elements)
            off = np.abs(got - want) / bf16_ulp(want)
            n_off = int(np.count_nonzero(off > 1.0 + 1e-9))
            note("  bf16 dZ elements beyond one ulp: %d of %d" % (n_off, off.size))
            assert n_off <= 1e-4 * off.size, (dl, n_off, off.max())
        # dW2 on those columns: float32 dlogits against the oracle's dW2;
        # bf16 dlogits (dW2 is then formed from the stored bf16 values)
        # against E^T times the oracle's dZ rounded the same way
        dw2 = out["dW2"][:, cidx].cpu().numpy().astype(np.float64)
        want_dw2 = ref["dW2"] if dl == "f32" else E.T @ want
        e = rel_l2(dw2, want_dw2, axis=0)
        assert e.max() <= 2e-3 and rel_l2(dw2, want_dw2) <= 2e-3, (dl, e.max())
        del out, dz
