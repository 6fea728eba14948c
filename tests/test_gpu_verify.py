"""GPU parity of dspark_verify_block against the CPU oracle (through the C ABI).

The GPU drafts the blocks (dspark_draft_block), then verifies them against
synthetic target logits; the oracle verifies the same drafted tokens with
the same logp and survival values (the GPU's, widened exactly), so the
comparison isolates the verification step.

Integer results are compared exactly, except where floating point decides
them by a hair: an accept test whose oracle margin |u p_d - p_t| / max is
below 1e-4 (the GPU takes p_t from float32 row sums), or a final draw whose
oracle top-two gap is below 1e-4 (the GPU's residual uses its own float32
draft row); such blocks are only checked for validity.
"""
import numpy as np
import pytest

import oracle
import synth
from _parity import note

pytestmark = pytest.mark.gpu

MARGIN = 1e-4
GAP = 1e-4


@pytest.fixture(scope="module")
def ops():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from semi_autoregressive_draft_markov_amd import binding, ops as _ops
    binding.load()
    return _ops


def make_target(inp, noise=0.4, seed=77):
    """Target logits [B, gamma+1, V]: the base logits plus noise at the gamma
    drafted positions, fresh logits at the bonus position (stored like U)."""
    rng = np.random.default_rng(seed)
    U = inp.as_f32(inp.U)
    t = np.empty((inp.B, inp.gamma + 1, inp.V), np.float32)
    t[:, :inp.gamma] = U + rng.standard_normal(U.shape, dtype=np.float32) * np.float32(noise)
    t[:, inp.gamma] = rng.standard_normal((inp.B, inp.V), dtype=np.float32) * np.float32(2.0)
    return synth.f32_to_bf16_bits(t) if inp.dtype == "bf16" else t


def run(ops, inp, target, tau, seed=5, offset=3):
    import torch
    t = synth.to_torch(inp)
    d = ops.draft_block(t["U"], t["h"], t["anchor"], t["W1"], t["W2"], t["w_conf"], t["temperature"],
                        seed=seed, offset=offset)
    tt = torch.as_tensor(target.view(np.int16) if inp.dtype == "bf16" else target).to(t["U"].device)
    if inp.dtype == "bf16":
        tt = tt.view(torch.bfloat16)
    v = ops.verify_block(t["U"], t["anchor"], t["W1"], t["W2"], tt, d["tokens"], d["logp"],
                         d["survival"], t["temperature"], threshold=tau, seed=seed, offset=offset)
    torch.cuda.synchronize()
    g = {k: d[k].cpu().numpy() for k in ("tokens", "logp", "survival")}
    for k in ("n_keep", "n_accept", "next_token", "accept_prob"):
        g[k] = v[k].cpu().numpy()
    g["_v"] = v
    return g


def check(inp, target, g, tau, seed=5, offset=3, label=""):
    ref = oracle.verify_block(inp, g["tokens"], g["logp"].astype(np.float64),
                              g["survival"].astype(np.float64), target, tau, seed=seed, offset=offset)
    assert np.array_equal(g["n_keep"], ref["keep"]), label
    close = 0
    for b in range(inp.B):
        if ref["margin"][b] < MARGIN:
            close += 1
            assert 0 <= g["n_accept"][b] <= g["n_keep"][b]
            continue
        assert g["n_accept"][b] == ref["accept"][b], (label, b, g["n_accept"][b], ref["accept"][b])
        if ref["gap"][b] < GAP:
            close += 1
            assert 0 <= g["next_token"][b] < inp.V
            continue
        assert g["next_token"][b] == ref["next"][b], (label, b, g["next_token"][b], ref["next"][b])
        tested = ~np.isnan(ref["accept_prob"][b])
        assert np.array_equal(tested, ~np.isnan(g["accept_prob"][b])), (label, b)
        assert np.allclose(g["accept_prob"][b][tested], ref["accept_prob"][b][tested], rtol=1e-3, atol=1e-6)
    assert close <= max(1, inp.B // 10), (label, close)
    note("%s: kept %s accepted %s" % (label, np.bincount(ref["keep"]).tolist(), np.bincount(ref["accept"]).tolist()))
    return ref


def small(**kw):
    base = dict(V=1000, r=64, d=32, gamma=5, B=40, dtype="bf16", head="markov", seed=41,
                u_std=2.0, w1_std=0.25, w2_std=0.25, wconf_std=0.3, h_std=1.0,
                anchors="uniform", temperature=[1.0] * 30 + [0.0] * 10)
    base.update(kw)
    return synth.make_inputs(**base)


@pytest.mark.parametrize("tau", [0.0, 0.25, 2.0])
def test_matrix_core_mixed_temperatures(ops, tau):
    inp = small()
    target = make_target(inp)
    note("case: verify mfma V1000 r64 B40 tau %g" % tau)
    g = run(ops, inp, target, tau)
    ref = check(inp, target, g, tau, label="tau %g" % tau)
    if tau == 0.0:
        assert (ref["keep"] == inp.gamma).all()
        assert ref["accept"].max() >= 2  # some acceptances happen
        assert (ref["accept"] < ref["keep"]).any()  # and some residual draws
    if tau == 2.0:
        assert (ref["keep"] == 0).all()


def test_rank256_ragged(ops):
    inp = small(V=2056, r=256, B=19, gamma=4, seed=42, temperature=1.0)
    target = make_target(inp, noise=0.2, seed=78)
    note("case: verify mfma V2056 r256 B19")
    check(inp, target, run(ops, inp, target, 0.125), 0.125, label="r256")


def test_vector_path_fp32(ops):
    inp = small(V=999, r=48, B=12, dtype="f32", seed=43, temperature=[1.0] * 8 + [0.0] * 4)
    target = make_target(inp, seed=79)
    note("case: verify vector fp32 V999 r48")
    check(inp, target, run(ops, inp, target, 0.25), 0.25, label="vector")


def test_bad_token_is_flagged(ops):
    import torch
    from semi_autoregressive_draft_markov_amd import binding
    inp = small(B=4, seed=44, temperature=1.0)
    target = make_target(inp, seed=80)
    t = synth.to_torch(inp)
    d = ops.draft_block(t["U"], t["h"], t["anchor"], t["W1"], t["W2"], t["w_conf"], t["temperature"])
    tok = d["tokens"].clone()
    tok[1, 2] = inp.V
    tt = torch.as_tensor(target.view(np.int16)).to(t["U"].device).view(torch.bfloat16)
    v = ops.verify_block(t["U"], t["anchor"], t["W1"], t["W2"], tt, tok, d["logp"], d["survival"],
                         t["temperature"], threshold=0.0)
    torch.cuda.synchronize()
    assert binding.dspark_read_device_error(v["_dims"], v["_ws"]) == 1
    assert v["next_token"][1].item() == -1 and v["n_keep"][1].item() == 0
    assert (v["next_token"][[0, 2, 3]] >= 0).all()
    assert torch.isnan(v["accept_prob"][1]).all()


def test_deterministic(ops):
    inp = small(seed=45)
    target = make_target(inp, seed=81)
    a = run(ops, inp, target, 0.25)
    b = run(ops, inp, target, 0.25)
    for k in ("n_keep", "n_accept", "next_token"):
        assert np.array_equal(a[k], b[k]), k
    assert np.array_equal(np.nan_to_num(a["accept_prob"], nan=-1), np.nan_to_num(b["accept_prob"], nan=-1))


def test_qwen3_4b_shape_every_block(ops):
    inp = synth.config_inputs(2)
    target = make_target(inp, noise=0.3, seed=82)
    note("case: verify qwen3-4b-shaped V151936 r256 B32")
    ref = check(inp, target, run(ops, inp, target, 0.0), 0.0, label="qwen3-4b")
    assert (ref["accept"] < ref["keep"]).any() and (ref["accept"] > 0).any()


def test_many_blocks(ops):
    # 130 blocks: several 16-block units in the draft-row kernel and one
    # final-draw workgroup per (block, chunk), each block's last one picking
    # its token
    inp = small(V=9000, r=64, gamma=4, B=130, seed=47, temperature=[1.0] * 90 + [0.0] * 40)
    target = make_target(inp, noise=0.3, seed=84)
    note("case: verify V9000 r64 B130")
    check(inp, target, run(ops, inp, target, 0.125), 0.125, label="many blocks")


def test_longest_block(ops):
    # gamma = 64: every lane of the decision wave holds a position, the
    # bonus row is the 65th; the target equals the base logits closely so
    # long accepted runs occur
    inp = small(V=520, r=32, gamma=64, B=6, seed=46, w1_std=0.05, w2_std=0.05,
                temperature=[1.0] * 4 + [0.0] * 2)
    target = make_target(inp, noise=0.05, seed=83)
    note("case: verify gamma 64")
    ref = check(inp, target, run(ops, inp, target, 0.0), 0.0, label="gamma 64")
    assert ref["accept"].max() >= 8
