"""GPU parity of dspark_draft_block against the CPU oracle (through the C ABI).

Sizes span several V tiles with ragged tails, padded block columns, both
heads, both dtypes, mixed temperatures, and the full workloads (all blocks
or a sample of blocks recomputed with their original noise).
"""
import itertools

import numpy as np
import pytest
from scipy import stats

import oracle
import synth
from _parity import check_draft, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from semi_autoregressive_draft_markov_amd import binding, ops as _ops
    binding.load()
    return _ops


MULTI, SINGLE = 1, 2  # per-step launches / single-launch kernel


def run_gpu(ops, inp, seed=0, offset=0, path=0):
    import torch
    from semi_autoregressive_draft_markov_amd import binding
    binding.dspark_set_option(binding.DSPARK_OPT_DRAFT_PATH, path)
    t = synth.to_torch(inp)
    out = ops.draft_block(t["U"], t["h"], t["anchor"], t["W1"], t["W2"], t["w_conf"],
                          t["temperature"], W_rnn=t["W_rnn"], seed=seed, offset=offset)
    torch.cuda.synchronize()
    res = {k: out[k].cpu().numpy() for k in ("tokens", "logp", "conf", "survival")}
    res["_out"] = out
    return res


def small(**kw):
    base = dict(V=1000, r=64, d=48, gamma=5, B=20, dtype="bf16", head="markov", seed=3,
                u_std=3.0, h_std=1.0, w1_std=0.25, w2_std=0.25, wconf_std=0.1, wrnn_std=0.1,
                anchors="uniform", temperature=1.0)
    base.update(kw)
    return synth.make_inputs(**base)


# -------------------------------------------------------------- small cases

@pytest.mark.parametrize("temp", [1.0, 0.0])
def test_tiny_fp32_block(ops, temp):
    inp = synth.config_inputs(1, temperature=temp)
    note("case: tiny fp32 V1024 r32 B4 T=%s" % temp)
    g = run_gpu(ops, inp, seed=0)
    check_draft(inp, g, 0, 0, label="tiny fp32")


@pytest.mark.parametrize("path", [MULTI, SINGLE])
def test_bf16_matrix_core_ragged_mixed_temperature(ops, path):
    # V = 1000: 4 workgroups, last one 232 columns; 64-column wave tiles with
    # a 40-column tail; B = 20 pads to 32 block columns.  Strong bias.
    temps = [1.0] * 8 + [0.0] * 6 + [0.7] * 6
    inp = small(temperature=temps)
    note("case: bf16 mfma V1000 r64 B20 mixed T path %d" % path)
    g = run_gpu(ops, inp, seed=11, offset=5, path=path)
    check_draft(inp, g, 11, 5, label="bf16 mfma ragged")


@pytest.mark.parametrize("gamma", [1, 2, 3])
def test_single_launch_short_blocks(ops, gamma):
    # the first and last steps of the single-launch loop (no grid barrier at
    # gamma = 1, one at gamma = 2) with two 16-block groups
    inp = small(V=1000, r=64, d=48, gamma=gamma, B=21, seed=30 + gamma,
                temperature=[1.0] * 15 + [0.0] * 6)
    note("case: bf16 single-launch short blocks gamma %d" % gamma)
    g = run_gpu(ops, inp, seed=6, offset=2, path=SINGLE)
    check_draft(inp, g, 6, 2, label="short blocks gamma %d" % gamma)


def test_single_launch_many_blocks(ops):
    # B = 300: E rows staged 16 blocks at a time (19 block groups, the last
    # one partial), the workgroup merge loops over 38 groups of 8 blocks
    temps = [1.0] * 150 + [0.0] * 100 + [0.8] * 50
    inp = small(V=4104, r=256, d=64, gamma=3, B=300, seed=34, temperature=temps)
    note("case: bf16 single-launch V4104 r256 B300")
    g = run_gpu(ops, inp, seed=8, offset=1, path=SINGLE)
    pick = np.array([0, 1, 15, 16, 149, 150, 255, 256, 287, 288, 298, 299])
    sub = synth.subset(inp, pick)
    check_draft(sub, {k: g[k][pick] for k in ("tokens", "logp", "conf", "survival")}, 8, 1,
                block_ids=pick, label="single launch B300")


def test_single_launch_longest_block(ops):
    # gamma = 64, the largest the C ABI accepts: 63 grid barriers, the
    # finish kernel's waves each take 8 positions
    inp = small(V=2048, r=64, d=48, gamma=64, B=5, seed=33, w1_std=0.05, w2_std=0.05,
                temperature=[1.0, 0.0, 1.0, 0.5, 1.0])
    note("case: bf16 single-launch gamma 64")
    g = run_gpu(ops, inp, seed=7, offset=3, path=SINGLE)
    check_draft(inp, g, 7, 3, label="single launch gamma 64")


@pytest.mark.parametrize("path", [MULTI, SINGLE])
@pytest.mark.parametrize("B", [1, 33])
def test_bf16_rank256_tail_columns(ops, B, path):
    inp = small(V=4104, r=256, d=64, gamma=7, B=B, seed=4)
    note("case: bf16 mfma V4104 r256 B%d path %d" % (B, path))
    g = run_gpu(ops, inp, seed=2, path=path)
    check_draft(inp, g, 2, 0, label="bf16 r256")


# bf16 with d % 8 == 0: joint projection on matrix cores (h columns hoisted
# out of the loop, ragged 32-row tiles, a d tail shorter than 32); f32 and
# d % 8 != 0: the vector projection
@pytest.mark.parametrize("dtype,V,r,d,B", [("bf16", 512, 32, 40, 10), ("f32", 512, 32, 40, 10),
                                           ("bf16", 1000, 64, 72, 37), ("bf16", 512, 32, 20, 5)])
def test_rnn_head_small(ops, dtype, V, r, d, B):
    temps = [1.0] * ((B + 1) // 2) + [0.0] * (B // 2)
    inp = small(V=V, r=r, d=d, gamma=4, B=B, head="rnn", dtype=dtype, seed=8,
                wrnn_std=0.3, temperature=temps)
    note("case: rnn %s V%d r%d d%d B%d" % (dtype, V, r, d, B))
    g = run_gpu(ops, inp, seed=6, offset=1)
    check_draft(inp, g, 6, 1, label="rnn " + dtype)


def test_vector_path_odd_shapes(ops):
    # V not a multiple of 8 and r not a multiple of 32: the plain vector path
    inp = small(V=999, r=48, d=20, gamma=3, B=6, seed=9)
    note("case: bf16 vector path V999 r48")
    g = run_gpu(ops, inp, seed=1)
    check_draft(inp, g, 1, 0, label="vector path")


def test_zero_confidence_weights(ops):
    inp = small(B=4, gamma=6)
    inp.w_conf = np.zeros_like(inp.w_conf)
    g = run_gpu(ops, inp)
    assert np.all(g["conf"] == 0.5)
    assert np.all(g["survival"] == (0.5 ** np.arange(1, 7))[None, :].astype(np.float32))


@pytest.mark.parametrize("path", [MULTI, SINGLE])
def test_deterministic(ops, path):
    inp = small(V=2048, r=128, B=24, seed=12)
    a = run_gpu(ops, inp, seed=3, path=path)
    b = run_gpu(ops, inp, seed=3, path=path)
    for k in ("tokens", "logp", "conf", "survival"):
        assert np.array_equal(a[k], b[k], equal_nan=True), k
    c = run_gpu(ops, inp, seed=3, offset=1, path=path)
    assert not np.array_equal(a["tokens"], c["tokens"])


def test_paths_agree(ops):
    # both drivers compute the same keys; tokens agree exactly and the
    # float outputs to rounding of the softmax normaliser
    inp = small(V=4104, r=256, d=64, gamma=7, B=40, seed=13, temperature=[1.0] * 30 + [0.0] * 10)
    a = run_gpu(ops, inp, seed=9, path=MULTI)
    b = run_gpu(ops, inp, seed=9, path=SINGLE)
    assert np.array_equal(a["tokens"], b["tokens"])
    assert np.allclose(a["logp"], b["logp"], rtol=0, atol=1e-5)
    assert np.array_equal(a["conf"], b["conf"]) or np.allclose(a["conf"], b["conf"], rtol=1e-6)


@pytest.mark.parametrize("path", [MULTI, SINGLE])
def test_out_of_range_anchor_is_flagged(ops, path):
    from semi_autoregressive_draft_markov_amd import binding
    inp = small(B=5)
    inp.anchor = np.array([3, inp.V, 7, -1, 0], np.int32)
    g = run_gpu(ops, inp, path=path)
    assert np.all(g["tokens"][[1, 3]] == -1)
    assert np.all(np.isnan(g["conf"][[1, 3]]))
    assert np.all(g["tokens"][[0, 2, 4]] >= 0)
    out = g["_out"]
    assert binding.dspark_read_device_error(out["_dims"], out["_ws"]) == 2
    good = synth.subset(inp, [0, 2, 4])
    check_draft(good, {k: g[k][[0, 2, 4]] for k in ("tokens", "logp", "conf", "survival")},
                0, 0, block_ids=[0, 2, 4], label="valid blocks")


@pytest.mark.parametrize("dtype,V,path", [("bf16", 8, MULTI), ("bf16", 8, SINGLE), ("f32", 4, MULTI)])
def test_sampler_law_on_gpu(ops, dtype, V, path):
    # GPU block frequencies follow the exact Eq 4 product (chi-square).
    gamma, n = 2, 60000
    inp = small(V=V, r=32, d=8, gamma=gamma, B=1, dtype=dtype, w1_std=0.5, w2_std=0.5,
                u_std=1.0, seed=5)
    if path == SINGLE:
        # the single-launch kernel holds per-block state in LDS: draw the
        # samples as 200 calls of 300 blocks with distinct noise offsets
        rep = synth.subset(inp, np.zeros(300, dtype=np.int64))
        toks = np.concatenate([run_gpu(ops, rep, seed=77, offset=o, path=path)["tokens"]
                               for o in range(n // 300)])
    else:
        rep = synth.subset(inp, np.zeros(n, dtype=np.int64))
        toks = run_gpu(ops, rep, seed=77, path=path)["tokens"]
    codes = toks[:, 0] * V + toks[:, 1]
    counts = np.bincount(codes, minlength=V * V)
    blocks = np.array(list(itertools.product(range(V), repeat=gamma)), np.int32)
    probs = np.exp(oracle.block_logprob(synth.subset(inp, np.zeros(len(blocks), np.int64)), blocks))
    exp = probs * n
    keep = exp > 5
    chi2 = (((counts - exp) ** 2) / exp)[keep].sum()
    p = stats.chi2.sf(chi2, keep.sum() - 1)
    assert p > 1e-4, (chi2, p)


# -------------------------------------------------------------- full sizes

@pytest.mark.parametrize("path", [MULTI, SINGLE])
def test_qwen3_4b_shape_all_blocks(ops, path):
    inp = synth.config_inputs(2)
    note("case: qwen3-4b-shaped V151936 r256 B32 (all blocks) path %d" % path)
    g = run_gpu(ops, inp, seed=0, path=path)
    info = check_draft(inp, g, 0, 0, label="qwen3-4b shape")
    note("  ties allowed: %d, max |dlogp| %.2e" % (info["ties"], info["logp_err"]))


@pytest.mark.parametrize("path", [MULTI, SINGLE])
def test_qwen3_4b_shape_strong_bias_all_blocks(ops, path):
    # W1, W2 ~ N(0, 0.25^2): the transition bias has std ~1 (r = 256), next
    # to U's 3, so every column -- the register tiles and the 20864 columns
    # past 131072 that the single-launch kernel holds in LDS fragments --
    # moves the argmax; sampled, greedy and tempered blocks
    temps = ([1.0, 0.0, 0.7, 1.0] * 8)[:32]
    inp = synth.config_inputs(2, w1_std=0.25, w2_std=0.25, temperature=temps, seed=1202)
    note("case: qwen3-4b-shaped strong bias V151936 r256 B32 (all blocks) path %d" % path)
    g = run_gpu(ops, inp, seed=5, offset=3, path=path)
    info = check_draft(inp, g, 5, 3, label="qwen3-4b shape strong bias")
    note("  ties allowed: %d, max |dlogp| %.2e" % (info["ties"], info["logp_err"]))


def plant_ties(inp, rng, cols_per_row):
    """Greedy blocks with W2 = 0: the bias is exactly 0 on both sides, so z
    = U exactly.  At every (block, position) the value 32 (above every
    N(0, 9) draw in bf16) is planted at the given columns; the argmax is
    then an exact tie whose lowest index must win."""
    U = inp.U.copy()
    top = synth.f32_to_bf16_bits(np.array([32.0], np.float32))[0] if inp.dtype == "bf16" else np.float32(32.0)
    want = np.zeros((inp.B, inp.gamma), np.int32)
    for b in range(inp.B):
        for k in range(inp.gamma):
            cols = cols_per_row(b, k, rng)
            U[b, k, cols] = top
            want[b, k] = min(cols)
    inp.U = U
    inp.W2 = np.zeros_like(inp.W2)
    inp.temperature = np.zeros(inp.B, np.float32)
    return want


@pytest.mark.parametrize("path", [MULTI, SINGLE])
def test_exact_ties_take_the_lowest_index(ops, path):
    # pairs of equal maxima: in one lane's columns, across lanes, across
    # waves and workgroups, and (single-launch kernel) between a register
    # tile column and an LDS-fragment column past 131072
    inp = synth.config_inputs(2, seed=1203)
    V = inp.V

    def cols(b, k, rng):
        kind = (b + k) % 5
        v = int(rng.integers(0, V - 70000))
        if kind == 0:
            return [v, v + 1]
        if kind == 1:
            return [v + 37, v + 5]
        if kind == 2:
            return [v + 64 * 9, v]
        if kind == 3:
            return [v + 60000, v + 3, v + 61000]
        return [int(rng.integers(131072, V)), int(rng.integers(0, 131072))]

    want = plant_ties(inp, np.random.default_rng(9), cols)
    note("case: qwen3-4b-shaped exact ties, greedy, W2 = 0, path %d" % path)
    g = run_gpu(ops, inp, seed=0, path=path)
    assert np.array_equal(g["tokens"], want), np.argwhere(g["tokens"] != want)[:5]
    check_draft(inp, g, 0, 0, label="exact ties")


def test_exact_ties_small_vocabulary(ops):
    # the per-step driver's vector path (f32) and a ragged bf16 tail
    for dtype, V in (("f32", 999), ("bf16", 1000)):
        inp = small(V=V, r=32 if dtype == "bf16" else 48, d=16, gamma=4, B=6, dtype=dtype, seed=61)
        want = plant_ties(inp, np.random.default_rng(10),
                          lambda b, k, rng: sorted(rng.choice(V, size=2 + (b % 2), replace=False)
                                                   .tolist(), reverse=True))
        note("case: exact ties %s V%d" % (dtype, V))
        g = run_gpu(ops, inp, seed=0)
        assert np.array_equal(g["tokens"], want), (dtype, np.argwhere(g["tokens"] != want)[:5])
        check_draft(inp, g, 0, 0, label="exact ties " + dtype)


def test_qwen3_4b_shape_mixed_temperature_single_launch(ops):
    # V = 151936: every wave of the single-launch kernel has its full
    # register tile and LDS fragment, so the branch-free statistics run;
    # sampled, greedy (zero noise) and tempered blocks in both 16-block
    # groups
    temps = ([1.0, 0.0, 0.7] * 8)[:24]
    inp = synth.config_inputs(2, B=24, temperature=temps, seed=1102)
    note("case: qwen3-4b-shaped V151936 r256 B24 mixed T single launch")
    g = run_gpu(ops, inp, seed=3, offset=1, path=SINGLE)
    info = check_draft(inp, g, 3, 1, label="qwen3-4b shape mixed T")
    note("  ties allowed: %d, max |dlogp| %.2e" % (info["ties"], info["logp_err"]))


def test_single_launch_dirty_reused_workspace(ops):
    # the workspace arrives with arbitrary contents (all bits set: argmax
    # keys that would beat every real key, barrier counters far past any
    # target) and is then reused by a call with fewer blocks and positions;
    # the kernel clears what it uses itself
    import torch
    from semi_autoregressive_draft_markov_amd import binding
    binding.dspark_set_option(binding.DSPARK_OPT_DRAFT_PATH, SINGLE)
    big = small(V=4104, r=256, d=64, gamma=6, B=28, seed=51, temperature=[1.0] * 20 + [0.0] * 8)
    tb = synth.to_torch(big)
    dims = ops.draft_dims(tb["U"], tb["h"], tb["W1"])
    ws = ops.workspace(dims, binding.DSPARK_CALL_DRAFT, tb["U"].device)
    ws.fill_(0xFF)
    note("case: single launch, workspace filled with 0xFF, V4104 B28 gamma6")
    out = ops.draft_block(tb["U"], tb["h"], tb["anchor"], tb["W1"], tb["W2"], tb["w_conf"], tb["temperature"],
                          seed=4, offset=2, ws=ws)
    torch.cuda.synchronize()
    check_draft(big, {k: out[k].cpu().numpy() for k in ("tokens", "logp", "conf", "survival")}, 4, 2,
                label="dirty workspace")
    sm = small(V=4104, r=256, d=64, gamma=3, B=9, seed=52)
    ts = synth.to_torch(sm)
    note("case: the same workspace again, V4104 B9 gamma3")
    out = ops.draft_block(ts["U"], ts["h"], ts["anchor"], ts["W1"], ts["W2"], ts["w_conf"], ts["temperature"],
                          seed=5, ws=ws)
    torch.cuda.synchronize()
    check_draft(sm, {k: out[k].cpu().numpy() for k in ("tokens", "logp", "conf", "survival")}, 5, 0,
                label="reused workspace")


def test_single_launch_barrier_time_out_is_reported(ops):
    # every grid-barrier wait forced to give up at once (the kernel's own
    # bounded waits, set from the host): the call completes, every block is
    # invalid and dspark_read_device_error reports the time-out; the next
    # call with the default limit is correct again
    import torch
    from semi_autoregressive_draft_markov_amd import binding
    inp = small(V=4104, r=256, d=64, gamma=4, B=12, seed=61)
    t = synth.to_torch(inp)
    binding.dspark_set_option(binding.DSPARK_OPT_DRAFT_PATH, SINGLE)
    binding.dspark_set_option(binding.DSPARK_OPT_BARRIER_SPIN, -1)
    try:
        note("case: single launch, barrier waits forced to give up, V4104 B12 gamma4")
        out = ops.draft_block(t["U"], t["h"], t["anchor"], t["W1"], t["W2"], t["w_conf"], t["temperature"], seed=6)
        torch.cuda.synchronize()
        assert (out["tokens"].cpu().numpy() == -1).all()
        assert np.isnan(out["survival"].cpu().numpy()).all()
        with pytest.raises(binding.DsparkError) as e:
            binding.dspark_read_device_error(out["_dims"], out["_ws"])
        assert e.value.status == binding.DSPARK_EDEVICE and "gave up" in str(e.value)
    finally:
        binding.dspark_set_option(binding.DSPARK_OPT_BARRIER_SPIN, 0)
    note("case: the same call with the default limit")
    g = run_gpu(ops, inp, seed=6, path=SINGLE)
    check_draft(inp, g, 6, 0, label="after forced time-out")
    assert binding.dspark_read_device_error(g["_out"]["_dims"], g["_out"]["_ws"]) == 0


@pytest.mark.parametrize("path", [MULTI, SINGLE])
def test_qwen3_14b_shape_all_blocks(ops, path):
    inp = synth.config_inputs(4)
    note("case: qwen3-14b-shaped V151936 r256 B256 half greedy (all blocks) path %d" % path)
    g = run_gpu(ops, inp, seed=0, path=path)
    info = check_draft(inp, g, 0, 0, label="qwen3-14b shape")
    note("  ties allowed: %d, max |dlogp| %.2e" % (info["ties"], info["logp_err"]))


def test_gemma4_rnn_shape_all_blocks(ops):
    inp = synth.config_inputs(5)
    note("case: gemma4-12b-shaped rnn V262144 r256 B128 (all blocks)")
    g = run_gpu(ops, inp, seed=0)
    info = check_draft(inp, g, 0, 0, label="gemma4 rnn shape")
    note("  ties allowed: %d, max |dlogp| %.2e" % (info["ties"], info["logp_err"]))
