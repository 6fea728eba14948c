"""The C-ABI library loads on the host and exports what include/dspark.h
declares; host-side argument checks return the documented statuses.  No
call here reaches the GPU (every checked call fails validation first)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*[a-zA-Z_][\w\s\*]*?\b(dspark_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    from semi_autoregressive_draft_markov_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from semi_autoregressive_draft_markov_amd import build
        build.build()
    return binding


def test_header_declares_the_boundary():
    names = declared_functions()
    for need in ("dspark_draft_block", "dspark_block_loss", "dspark_block_loss_backward",
                 "dspark_verify_block", "dspark_workspace_size",
                 "dspark_read_device_error", "dspark_last_error", "dspark_version"):
        assert need in names


def test_library_exports_every_declared_symbol(lib):
    so = ctypes.CDLL(lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(so, name), name


def test_version_and_workspace_sizes(lib):
    assert lib.dspark_version() == 1
    d = lib.make_dims(151936, 256, 2560, 7, 32)
    ws = lib.dspark_workspace_size(d, lib.DSPARK_CALL_DRAFT)
    assert ws > 0 and ws % 256 == 0
    assert lib.dspark_workspace_size(lib.make_dims(1, 256, 2560, 7, 32), 0) == 0
    assert lib.dspark_workspace_size(d, 7) == 0
    wb = lib.dspark_workspace_size(lib.make_dims(151936, 256, 4096, 7, 1024),
                                   lib.DSPARK_CALL_LOSS_BACKWARD)
    assert wb > 0 and wb % 256 == 0
    wv = lib.dspark_workspace_size(d, lib.DSPARK_CALL_VERIFY)
    assert wv > 0 and wv % 256 == 0


BAD_DIMS = [
    (dict(V=1), "V"), (dict(r=0), "r"), (dict(r=2048), "r"), (dict(d=0), "d"),
    (dict(gamma=0), "gamma"), (dict(gamma=65), "gamma"), (dict(B=0), "B"),
    (dict(dtype=5), "dtype"), (dict(head=9), "head"),
]


@pytest.mark.parametrize("bad,word", BAD_DIMS)
def test_draft_rejects_bad_dims(lib, bad, word):
    kw = dict(V=1000, r=64, d=32, gamma=7, B=4, dtype=1, head=0)
    kw.update(bad)
    d = lib.dspark_dims(kw["V"], kw["r"], kw["d"], kw["gamma"], kw["B"], kw["dtype"], kw["head"])
    with pytest.raises(lib.DsparkError) as e:
        lib.dspark_draft_block(d, *([8] * 8), 0, 0, *([256] * 5), workspace_bytes=1 << 30, stream=0)
    assert e.value.status == lib.DSPARK_EINVAL
    assert word in lib.dspark_last_error()


def test_draft_rejects_null_pointers_and_small_workspace(lib):
    d = lib.make_dims(1000, 64, 32, 7, 4)
    ptrs = [256] * 8
    for i, name in enumerate(["U", "h", "anchor", "W1", "W2", "w_conf"]):
        p = list(ptrs)
        p[i if i < 6 else i] = None
        with pytest.raises(lib.DsparkError) as e:
            lib.dspark_draft_block(d, *p, 0, 0, *([256] * 5), workspace_bytes=1 << 30, stream=0)
        assert e.value.status == lib.DSPARK_EINVAL and name in str(e.value)
    # RNN head needs W_rnn
    drnn = lib.make_dims(1000, 64, 32, 7, 4, head="rnn")
    p = list(ptrs)
    p[6] = None
    with pytest.raises(lib.DsparkError) as e:
        lib.dspark_draft_block(drnn, *p, 0, 0, *([256] * 5), workspace_bytes=1 << 30, stream=0)
    assert "W_rnn" in str(e.value)
    need = lib.dspark_workspace_size(d, lib.DSPARK_CALL_DRAFT)
    with pytest.raises(lib.DsparkError) as e:
        lib.dspark_draft_block(d, *ptrs, 0, 0, *([256] * 5), workspace_bytes=need - 1, stream=0)
    assert e.value.status == lib.DSPARK_EWORKSPACE
    with pytest.raises(lib.DsparkError) as e:
        lib.dspark_draft_block(d, *ptrs, 0, 0, *([256] * 4), 128, workspace_bytes=need, stream=0)
    assert e.value.status == lib.DSPARK_EINVAL and "aligned" in str(e.value)


def test_noise_rejects_bad_ranges(lib):
    for v0, n in ((-1, 4), (0, -1), ((1 << 31) - 2, 4)):
        with pytest.raises(lib.DsparkError) as e:
            lib.dspark_noise(0, 0, 0, 0, v0, n, stream=0)
        assert e.value.status == lib.DSPARK_EINVAL
    lib.dspark_noise(0, 0, 0, 0, 0, 0, stream=0)  # n = 0: nothing to do, no device work


def test_noalloc_draft_refuses_a_problem_beyond_its_scratch(lib):
    dims = lib.make_dims(151936, 256, 2560, 64, 1024)
    assert lib.dspark_workspace_size(dims, lib.DSPARK_CALL_DRAFT) > (32 << 20)
    with pytest.raises(lib.DsparkError) as e:
        lib.dspark_draft_block_noalloc(dims, *([256] * 8), 0, 0, *([256] * 4), stream=0)
    assert e.value.status == lib.DSPARK_EWORKSPACE and "scratch" in str(e.value)
    with pytest.raises(lib.DsparkError) as e:
        lib.dspark_draft_block_noalloc(lib.make_dims(1, 256, 2560, 7, 32), *([256] * 8), 0, 0,
                                       *([256] * 4), stream=0)
    assert e.value.status == lib.DSPARK_EINVAL


def test_read_device_error_rejects_null(lib):
    d = lib.make_dims(1000, 64, 32, 7, 4)
    st = lib.load().dspark_read_device_error(ctypes.byref(d), None, None, None)
    assert st == lib.DSPARK_EINVAL


def test_product_path_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "semi_autoregressive_draft_markov_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn)).read()
                assert not re.search(r"\boracle\b", text.replace("the oracle", "")), fn


def test_set_option_validates(lib):
    for opt, good, bad in ((lib.DSPARK_OPT_DRAFT_PATH, (0, 1, 2), (-1, 3)),
                           (lib.DSPARK_OPT_BARRIER_SPIN, (0, 100, -1), (-2,))):
        for v in good:
            lib.dspark_set_option(opt, v)
        for v in bad:
            with pytest.raises(lib.DsparkError) as e:
                lib.dspark_set_option(opt, v)
            assert e.value.status == lib.DSPARK_EINVAL
    lib.dspark_set_option(lib.DSPARK_OPT_DRAFT_PATH, 0)
    lib.dspark_set_option(lib.DSPARK_OPT_BARRIER_SPIN, 0)
    # the cooperative-launch option (formerly 2) no longer exists
    with pytest.raises(lib.DsparkError):
        lib.dspark_set_option(2, 0)
    with pytest.raises(lib.DsparkError) as e:
        lib.dspark_set_option(99, 0)
    assert "unknown option" in str(e.value)


def _loss_call(lib, d, ptr=256, **over):
    args = dict(U=ptr, T_logits=ptr, h=ptr, anchor=ptr, labels=ptr, W1=ptr, W2=ptr, w_conf=ptr,
                alpha=None, pos_weight=None, loss4=ptr, c_star=ptr, conf=None, dlogits=None,
                dlogits_dtype="f32", dW2=None, dconf_logit=None, workspace=ptr)
    args.update(over)
    wsb = over.pop("workspace_bytes", 1 << 40)
    args.pop("workspace_bytes", None)
    lib.dspark_block_loss(d, **args, workspace_bytes=wsb, stream=0)


def test_loss_rejects_bad_arguments(lib):
    d = lib.make_dims(1000, 64, 32, 7, 4)
    for name in ("U", "T_logits", "h", "anchor", "labels", "W1", "W2", "w_conf", "loss4",
                 "c_star", "workspace"):
        with pytest.raises(lib.DsparkError) as e:
            _loss_call(lib, d, **{name: None})
        assert e.value.status == lib.DSPARK_EINVAL and name in str(e.value)
    with pytest.raises(lib.DsparkError) as e:
        _loss_call(lib, d, dW2=256)
    assert e.value.status == lib.DSPARK_EINVAL and "dlogits" in str(e.value)
    with pytest.raises(lib.DsparkError) as e:
        _loss_call(lib, d, dlogits=256, dlogits_dtype=7)
    assert e.value.status == lib.DSPARK_EINVAL
    need = lib.dspark_workspace_size(d, lib.DSPARK_CALL_LOSS)
    with pytest.raises(lib.DsparkError) as e:
        _loss_call(lib, d, workspace_bytes=need - 1)
    assert e.value.status == lib.DSPARK_EWORKSPACE
    with pytest.raises(lib.DsparkError) as e:
        _loss_call(lib, lib.make_dims(1000, 64, 32, 7, 4, head="rnn"))
    assert e.value.status == lib.DSPARK_EUNSUPPORTED
    # bf16 matrix-core path needs 16-byte aligned streams
    with pytest.raises(lib.DsparkError) as e:
        _loss_call(lib, lib.make_dims(1024, 64, 32, 7, 4), U=258)
    assert e.value.status == lib.DSPARK_EUNSUPPORTED


def _bwd_call(lib, d, ptr=256, **over):
    args = dict(dlogits=ptr, dlogits_dtype="bf16", dconf_logit=ptr, h=ptr, anchor=ptr, labels=ptr,
                W1=ptr, W2=ptr, w_conf=ptr, dW1=ptr, dw_conf=ptr, dh=ptr, workspace=ptr)
    wsb = over.pop("workspace_bytes", 1 << 40)
    args.update(over)
    lib.dspark_block_loss_backward(d, **args, workspace_bytes=wsb, stream=0)


def test_loss_backward_rejects_bad_arguments(lib):
    d = lib.make_dims(1000, 64, 32, 7, 4)
    for name in ("anchor", "labels", "W1", "W2", "w_conf", "workspace"):
        with pytest.raises(lib.DsparkError) as e:
            _bwd_call(lib, d, **{name: None})
        assert e.value.status == lib.DSPARK_EINVAL and name in str(e.value)
    # each output names the input it needs
    for over, word in ((dict(dlogits=None), "dlogits"), (dict(dconf_logit=None), "dconf_logit"),
                       (dict(h=None), "h (needed")):
        with pytest.raises(lib.DsparkError) as e:
            _bwd_call(lib, d, **over)
        assert e.value.status == lib.DSPARK_EINVAL and word in str(e.value)
    with pytest.raises(lib.DsparkError) as e:
        _bwd_call(lib, d, dlogits_dtype=7)
    assert e.value.status == lib.DSPARK_EINVAL
    need = lib.dspark_workspace_size(d, lib.DSPARK_CALL_LOSS_BACKWARD)
    with pytest.raises(lib.DsparkError) as e:
        _bwd_call(lib, d, workspace_bytes=need - 1)
    assert e.value.status == lib.DSPARK_EWORKSPACE
    with pytest.raises(lib.DsparkError) as e:
        _bwd_call(lib, lib.make_dims(1000, 64, 32, 7, 4, head="rnn"))
    assert e.value.status == lib.DSPARK_EUNSUPPORTED
    with pytest.raises(lib.DsparkError) as e:
        _bwd_call(lib, d, dlogits=258)
    assert e.value.status == lib.DSPARK_EUNSUPPORTED
    with pytest.raises(lib.DsparkError) as e:
        _bwd_call(lib, d, dW1=258)
    assert e.value.status == lib.DSPARK_EINVAL


def _verify_call(lib, d, ptr=256, **over):
    args = dict(U=ptr, anchor=ptr, W1=ptr, W2=ptr, T_logits=ptr, tokens=ptr, logp=ptr,
                survival=ptr, temperature=ptr, threshold=0.5, seed=0, offset=0, n_keep=ptr,
                n_accept=ptr, next_token=ptr, accept_prob=None, workspace=ptr)
    wsb = over.pop("workspace_bytes", 1 << 40)
    args.update(over)
    lib.dspark_verify_block(d, **args, workspace_bytes=wsb, stream=0)


def test_verify_rejects_bad_arguments(lib):
    d = lib.make_dims(1000, 64, 1, 7, 4)
    for name in ("U", "anchor", "W1", "W2", "T_logits", "tokens", "logp", "survival",
                 "temperature", "n_keep", "n_accept", "next_token", "workspace"):
        with pytest.raises(lib.DsparkError) as e:
            _verify_call(lib, d, **{name: None})
        assert e.value.status == lib.DSPARK_EINVAL and name in str(e.value)
    with pytest.raises(lib.DsparkError) as e:
        _verify_call(lib, d, threshold=float("nan"))
    assert e.value.status == lib.DSPARK_EINVAL
    need = lib.dspark_workspace_size(d, lib.DSPARK_CALL_VERIFY)
    with pytest.raises(lib.DsparkError) as e:
        _verify_call(lib, d, workspace_bytes=need - 1)
    assert e.value.status == lib.DSPARK_EWORKSPACE
    with pytest.raises(lib.DsparkError) as e:
        _verify_call(lib, lib.make_dims(1000, 64, 1, 7, 4, head="rnn"))
    assert e.value.status == lib.DSPARK_EUNSUPPORTED
    with pytest.raises(lib.DsparkError) as e:
        _verify_call(lib, d, U=258)
    assert e.value.status == lib.DSPARK_EUNSUPPORTED
    with pytest.raises(lib.DsparkError) as e:
        _verify_call(lib, d, logp=258)
    assert e.value.status == lib.DSPARK_EINVAL
