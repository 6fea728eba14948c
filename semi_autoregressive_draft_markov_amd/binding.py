"""ctypes binding of libdspark.so (include/dspark.h), same names as the C ABI.

Argument marshalling only: tensors are passed as raw device pointers, every
step of the computation runs in the HIP library.  There is no fallback: if
the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build, or another build of the same sources named by
# DSPARK_LIBRARY (e.g. one compiled with host sanitizers)
LIB_PATH = os.environ.get("DSPARK_LIBRARY") or os.path.join(HERE, "libdspark.so")

DSPARK_OK, DSPARK_EINVAL, DSPARK_EUNSUPPORTED, DSPARK_EWORKSPACE, DSPARK_EDEVICE = range(5)
DSPARK_F32, DSPARK_BF16 = 0, 1
DSPARK_HEAD_MARKOV, DSPARK_HEAD_RNN = 0, 1
DSPARK_CALL_DRAFT, DSPARK_CALL_LOSS, DSPARK_CALL_LOSS_BACKWARD, DSPARK_CALL_VERIFY = 0, 1, 2, 3
DSPARK_OPT_DRAFT_PATH = 1
DSPARK_OPT_BARRIER_SPIN = 3

STATUS_NAMES = {0: "DSPARK_OK", 1: "DSPARK_EINVAL", 2: "DSPARK_EUNSUPPORTED",
                3: "DSPARK_EWORKSPACE", 4: "DSPARK_EDEVICE"}


class DsparkError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, status), message))
        self.status = status


class dspark_dims(ctypes.Structure):
    _fields_ = [("V", ctypes.c_int32), ("r", ctypes.c_int32), ("d", ctypes.c_int32),
                ("gamma", ctypes.c_int32), ("B", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("head", ctypes.c_int32)]


def make_dims(V, r, d, gamma, B, dtype="bf16", head="markov") -> dspark_dims:
    dt = {"f32": DSPARK_F32, "bf16": DSPARK_BF16}.get(dtype, dtype)
    hd = {"markov": DSPARK_HEAD_MARKOV, "rnn": DSPARK_HEAD_RNN}.get(head, head)
    return dspark_dims(V, r, d, gamma, B, dt, hd)


_lib = None


def load() -> ctypes.CDLL:
    """Load libdspark.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("%s is not built: run semi_autoregressive_draft_markov_amd.build.build()" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, U64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t
    D = ctypes.POINTER(dspark_dims)
    lib.dspark_workspace_size.argtypes = [D, ctypes.c_int]
    lib.dspark_workspace_size.restype = SZ
    lib.dspark_draft_block.argtypes = [D] + [P] * 8 + [U64, U64] + [P] * 5 + [SZ, P]
    lib.dspark_draft_block.restype = ctypes.c_int
    lib.dspark_draft_block_noalloc.argtypes = [D] + [P] * 8 + [U64, U64] + [P] * 4 + [P]
    lib.dspark_draft_block_noalloc.restype = ctypes.c_int
    lib.dspark_block_loss.argtypes = [D] + [P] * 13 + [P, I32, P, P, P, SZ, P]
    lib.dspark_block_loss.restype = ctypes.c_int
    lib.dspark_block_loss_backward.argtypes = [D, P, I32] + [P] * 11 + [SZ, P]
    lib.dspark_block_loss_backward.restype = ctypes.c_int
    lib.dspark_verify_block.argtypes = [D] + [P] * 9 + [ctypes.c_float, U64, U64] + [P] * 5 + [SZ, P]
    lib.dspark_verify_block.restype = ctypes.c_int
    F = ctypes.c_float
    lib.dspark_sts_calibrate.argtypes = [I32, I32, P, P, P, I32, I32, P, P, P]
    lib.dspark_sts_calibrate.restype = ctypes.c_int
    lib.dspark_schedule_prefixes.argtypes = [I32, I32, P, P, I32, P, P]
    lib.dspark_schedule_prefixes.restype = ctypes.c_int
    U32 = ctypes.c_uint32
    lib.dspark_noise.argtypes = [U64, U64, U32, U32, I32, I32, P, P, P, P, P]
    lib.dspark_noise.restype = ctypes.c_int
    lib.dspark_read_device_error.argtypes = [D, P, ctypes.POINTER(I32), P]
    lib.dspark_read_device_error.restype = ctypes.c_int
    lib.dspark_set_option.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.dspark_set_option.restype = ctypes.c_int
    lib.dspark_profile_enable.argtypes = [ctypes.c_int]
    lib.dspark_profile_enable.restype = ctypes.c_int
    lib.dspark_profile_read.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(I32)]
    lib.dspark_profile_read.restype = ctypes.c_int
    lib.dspark_profile_read_each.argtypes = [P, I32, ctypes.POINTER(I32)]
    lib.dspark_profile_read_each.restype = ctypes.c_int
    lib.dspark_draft_kernel_name.argtypes = [D]
    lib.dspark_draft_kernel_name.restype = ctypes.c_char_p
    lib.dspark_last_error.argtypes = []
    lib.dspark_last_error.restype = ctypes.c_char_p
    lib.dspark_version.argtypes = []
    lib.dspark_version.restype = ctypes.c_int
    _lib = lib
    return lib


def _p(t) -> Optional[int]:
    """Device (or host) address of a tensor / ctypes buffer / int, or NULL."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    return ctypes.addressof(t)


def _nbytes(t) -> int:
    if t is None:
        return 0
    if hasattr(t, "numel"):
        return t.numel() * t.element_size()
    return ctypes.sizeof(t)


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != DSPARK_OK:
        raise DsparkError(status, load().dspark_last_error().decode())


def dspark_version() -> int:
    return load().dspark_version()


def dspark_draft_kernel_name(dims: dspark_dims) -> str:
    return load().dspark_draft_kernel_name(ctypes.byref(dims)).decode()


def dspark_last_error() -> str:
    return load().dspark_last_error().decode()


def dspark_workspace_size(dims: dspark_dims, which: int) -> int:
    return load().dspark_workspace_size(ctypes.byref(dims), which)


def dspark_draft_block(dims, U, h, anchor, W1, W2, w_conf, W_rnn, temperature, seed, offset,
                       tokens, logp, conf, survival, workspace, workspace_bytes=None,
                       stream=None):
    nbytes = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    _check(load().dspark_draft_block(
        ctypes.byref(dims), _p(U), _p(h), _p(anchor), _p(W1), _p(W2), _p(w_conf), _p(W_rnn),
        _p(temperature), seed, offset, _p(tokens), _p(logp), _p(conf), _p(survival),
        _p(workspace), nbytes, _stream(stream)))


def dspark_draft_block_noalloc(dims, U, h, anchor, W1, W2, w_conf, W_rnn, temperature, seed, offset,
                               tokens, logp, conf, survival, stream=None):
    _check(load().dspark_draft_block_noalloc(
        ctypes.byref(dims), _p(U), _p(h), _p(anchor), _p(W1), _p(W2), _p(w_conf), _p(W_rnn),
        _p(temperature), seed, offset, _p(tokens), _p(logp), _p(conf), _p(survival), _stream(stream)))


def dspark_block_loss(dims, U, T_logits, h, anchor, labels, W1, W2, w_conf, alpha, pos_weight,
                      loss4, c_star, conf, dlogits, dlogits_dtype, dW2, dconf_logit,
                      workspace, workspace_bytes=None, stream=None):
    """alpha and pos_weight are HOST float32 sequences (or None)."""
    a = None if alpha is None else (ctypes.c_float * 3)(*alpha)
    pw = None if pos_weight is None else (ctypes.c_float * len(pos_weight))(*pos_weight)
    nbytes = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    _check(load().dspark_block_loss(
        ctypes.byref(dims), _p(U), _p(T_logits), _p(h), _p(anchor), _p(labels), _p(W1), _p(W2),
        _p(w_conf), _p(a), _p(pw), _p(loss4), _p(c_star), _p(conf), _p(dlogits),
        {"f32": DSPARK_F32, "bf16": DSPARK_BF16}.get(dlogits_dtype, dlogits_dtype),
        _p(dW2), _p(dconf_logit), _p(workspace), nbytes, _stream(stream)))


def dspark_block_loss_backward(dims, dlogits, dlogits_dtype, dconf_logit, h, anchor, labels, W1,
                               W2, w_conf, dW1, dw_conf, dh, workspace, workspace_bytes=None,
                               stream=None):
    nbytes = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    _check(load().dspark_block_loss_backward(
        ctypes.byref(dims), _p(dlogits),
        {"f32": DSPARK_F32, "bf16": DSPARK_BF16}.get(dlogits_dtype, dlogits_dtype),
        _p(dconf_logit), _p(h), _p(anchor), _p(labels), _p(W1), _p(W2), _p(w_conf), _p(dW1),
        _p(dw_conf), _p(dh), _p(workspace), nbytes, _stream(stream)))


def dspark_verify_block(dims, U, anchor, W1, W2, T_logits, tokens, logp, survival, temperature,
                        threshold, seed, offset, n_keep, n_accept, next_token, accept_prob,
                        workspace, workspace_bytes=None, stream=None):
    nbytes = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    _check(load().dspark_verify_block(
        ctypes.byref(dims), _p(U), _p(anchor), _p(W1), _p(W2), _p(T_logits), _p(tokens), _p(logp),
        _p(survival), _p(temperature), float(threshold), seed, offset, _p(n_keep), _p(n_accept),
        _p(next_token), _p(accept_prob), _p(workspace), nbytes, _stream(stream)))


def _host(a, dtype):
    import numpy as np
    return np.ascontiguousarray(a, dtype=dtype)


def dspark_sts_calibrate(conf_logit, accepted, grid=None, bins: int = 15):
    """HOST arrays: conf_logit [N, gamma], accepted [N]; returns (temperature,
    ece_before, ece_after) as float32 numpy arrays of length gamma."""
    import numpy as np
    a = _host(conf_logit, np.float32)
    acc = _host(accepted, np.int32)
    N, gamma = a.shape
    g = None if grid is None else _host(grid, np.float32)
    t = np.zeros(gamma, np.float32)
    eb = np.zeros(gamma, np.float32)
    ea = np.zeros(gamma, np.float32)
    _check(load().dspark_sts_calibrate(N, gamma, a.ctypes.data, acc.ctypes.data,
                                       None if g is None else g.ctypes.data,
                                       0 if g is None else len(g), bins, t.ctypes.data,
                                       eb.ctypes.data, ea.ctypes.data))
    return t, eb, ea


def dspark_schedule_prefixes(survival, sps):
    """HOST arrays: survival [R, gamma], sps [T + 1]; returns (length [R], theta)."""
    import numpy as np
    s = _host(survival, np.float32)
    sp = _host(sps, np.float32)
    R, gamma = s.shape
    length = np.zeros(R, np.int32)
    th = ctypes.c_float(0)
    _check(load().dspark_schedule_prefixes(R, gamma, s.ctypes.data, sp.ctypes.data, len(sp) - 1,
                                           length.ctypes.data, ctypes.addressof(th)))
    return length, th.value


def dspark_noise(seed, offset, c1, c2, v0, n, words_in=None, words=None, gumbel=None,
                 gumbel_log2=None, stream=None):
    """Device Philox words and Gumbel transforms (see include/dspark.h);
    tensors are device buffers of n elements, each optional."""
    _check(load().dspark_noise(seed, offset, c1, c2, v0, n, _p(words_in), _p(words), _p(gumbel),
                               _p(gumbel_log2), _stream(stream)))


def dspark_read_device_error(dims, workspace, stream=None) -> int:
    code = ctypes.c_int32(-1)
    _check(load().dspark_read_device_error(ctypes.byref(dims), _p(workspace),
                                           ctypes.byref(code), _stream(stream)))
    return code.value


def dspark_profile_enable(enable: bool) -> None:
    _check(load().dspark_profile_enable(1 if enable else 0))


def dspark_profile_read():
    """(summed milliseconds, launch count) of the dominant kernel since the last read."""
    ms = ctypes.c_float(0)
    n = ctypes.c_int32(0)
    _check(load().dspark_profile_read(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def dspark_profile_read_each(capacity: int = 4096):
    """Milliseconds of each timed launch since the last read, in recording
    order (a list of floats)."""
    buf = (ctypes.c_float * max(capacity, 1))()
    n = ctypes.c_int32(0)
    _check(load().dspark_profile_read_each(buf, capacity, ctypes.byref(n)))
    return [buf[i] for i in range(n.value)]


def dspark_set_option(option: int, value: int) -> None:
    _check(load().dspark_set_option(option, value))
