"""GPU test of the allocation-free drafting entry point: through the C ABI,
dspark_draft_block_noalloc must give exactly what dspark_draft_block gives
with a caller workspace, on consecutive calls that share the library's
scratch -- a large call first, then a smaller one that inherits its
contents -- on the single-launch kernel and on the per-step driver; a
problem larger than the built-in scratch is refused."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

OUTS = ("tokens", "logp", "conf", "survival")


@pytest.fixture(scope="module")
def lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from semi_autoregressive_draft_markov_amd import binding
    binding.load()
    return binding


def both(lib, inp, seed, offset, path):
    import torch
    from semi_autoregressive_draft_markov_amd import ops
    lib.dspark_set_option(lib.DSPARK_OPT_DRAFT_PATH, path)
    t = synth.to_torch(inp)
    dims = ops.draft_dims(t["U"], t["h"], t["W1"], t["W_rnn"])
    B, g = inp.B, inp.gamma

    def outs():
        return dict(tokens=torch.full((B, g), -7, dtype=torch.int32, device="cuda"),
                    **{k: torch.full((B, g), 7.0, dtype=torch.float32, device="cuda") for k in OUTS[1:]})

    ref, got = outs(), outs()
    ws = ops.workspace(dims, lib.DSPARK_CALL_DRAFT, t["U"].device)
    lib.dspark_draft_block(dims, t["U"], t["h"], t["anchor"], t["W1"], t["W2"], t["w_conf"], t["W_rnn"],
                           t["temperature"], seed, offset, ref["tokens"], ref["logp"], ref["conf"],
                           ref["survival"], ws)
    lib.dspark_draft_block_noalloc(dims, t["U"], t["h"], t["anchor"], t["W1"], t["W2"], t["w_conf"],
                                   t["W_rnn"], t["temperature"], seed, offset, got["tokens"], got["logp"],
                                   got["conf"], got["survival"])
    torch.cuda.synchronize()
    lib.dspark_set_option(lib.DSPARK_OPT_DRAFT_PATH, 0)
    for k in OUTS:
        a, b = ref[k].cpu().numpy(), got[k].cpu().numpy()
        assert np.array_equal(a, b, equal_nan=True), (k, np.argwhere(a != b)[:5])
    return ref["tokens"].cpu().numpy()


@pytest.mark.parametrize("path", [1, 2])  # per-step launches / single-launch kernel
def test_noalloc_matches_workspace_call_twice(lib, path):
    big = synth.config_inputs(2, w1_std=0.25, w2_std=0.25, temperature=[1.0, 0.0, 0.7, 1.0] * 8, seed=1301)
    print("case: no-alloc qwen3-4b-shaped B32 path %d" % path, flush=True)
    tok = both(lib, big, seed=3, offset=2, path=path)
    assert (tok >= 0).all()
    small = synth.make_inputs(V=4104, r=256, d=64, gamma=3, B=9, dtype="bf16", seed=1302, w1_std=0.25,
                              w2_std=0.25, anchors="uniform", temperature=[1.0] * 5 + [0.0] * 4)
    print("case: no-alloc V4104 B9 gamma3 path %d (after the larger call)" % path, flush=True)
    both(lib, small, seed=4, offset=0, path=path)


def test_noalloc_rnn_head_then_smaller(lib):
    a = synth.make_inputs(V=1000, r=64, d=72, gamma=4, B=37, dtype="bf16", head="rnn", seed=1303,
                          wrnn_std=0.3, w1_std=0.25, w2_std=0.25, anchors="uniform")
    print("case: no-alloc rnn V1000 B37", flush=True)
    both(lib, a, seed=1, offset=1, path=0)
    b = synth.make_inputs(V=512, r=32, d=40, gamma=2, B=5, dtype="bf16", head="rnn", seed=1304,
                          wrnn_std=0.3, w1_std=0.25, w2_std=0.25, anchors="uniform")
    print("case: no-alloc rnn V512 B5", flush=True)
    both(lib, b, seed=2, offset=0, path=0)


def test_noalloc_refuses_a_problem_beyond_its_scratch(lib):
    dims = lib.make_dims(151936, 256, 2560, 64, 1024)
    assert lib.dspark_workspace_size(dims, lib.DSPARK_CALL_DRAFT) > (32 << 20)
    with pytest.raises(lib.DsparkError) as e:
        lib.dspark_draft_block_noalloc(dims, *([256] * 8), 0, 0, *([256] * 4), stream=0)
    assert e.value.status == lib.DSPARK_EWORKSPACE and "scratch" in str(e.value)
