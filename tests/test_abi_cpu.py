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
    for need in ("dspark_draft_block", "dspark_block_loss", "dspark_workspace_size",
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
