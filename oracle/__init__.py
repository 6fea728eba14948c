"""CPU reference ("oracle") for the DSpark sequential head: ctypes front end.

TEST INFRASTRUCTURE ONLY.  Only tests/, the package smoke check and the
benchmark's CPU-baseline leg import this module; the product path never does,
and this module never imports the product package.  The arithmetic lives in
dspark_oracle.c (plain C, double precision); this file only builds that
library with gcc, marshals numpy arrays and returns numpy results.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dspark_oracle.c")
# the in-tree build, or another build of dspark_oracle.c named by
# DSPARK_ORACLE_LIBRARY (e.g. one compiled with sanitizers)
_LIB = os.environ.get("DSPARK_ORACLE_LIBRARY") or os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile dspark_oracle.c with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-Wall", "-Wextra", "-Wno-unused-parameter",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        U64 = ctypes.c_uint64
        lib.oracle_philox4x32_10.argtypes = [P, P, P]
        lib.oracle_philox4x32_10.restype = None
        lib.oracle_uniform.argtypes = [U64, U64, I, I, I]
        lib.oracle_uniform.restype = ctypes.c_double
        lib.oracle_gumbel.argtypes = [U64, U64, I, I, I]
        lib.oracle_gumbel.restype = ctypes.c_double
        lib.oracle_draft_block.argtypes = [I, I, I, I, I, I, I] + [P] * 8 + [U64, U64] + [P] * 8 + [I]
        lib.oracle_draft_block.restype = I
        lib.oracle_block_logprob.argtypes = [I, I, I, I, I, I, I] + [P] * 8 + [P, I]
        lib.oracle_block_logprob.restype = I
        lib.oracle_block_loss.argtypes = ([I, I, I, I, I, I] + [P] * 10 + [P, ctypes.c_int64]
                                          + [P, ctypes.c_int32] + [P] * 9 + [I])
        lib.oracle_block_loss.restype = I
        lib.oracle_block_loss_backward.argtypes = [I, I, I, I, I, I] + [P] * 11 + [I]
        lib.oracle_block_loss_backward.restype = I
        D = ctypes.c_double
        lib.oracle_verify_uniform.argtypes = [U64, U64, I, I]
        lib.oracle_verify_uniform.restype = D
        lib.oracle_verify_gumbel.argtypes = [U64, U64, I, I, I]
        lib.oracle_verify_gumbel.restype = D
        lib.oracle_verify_block.argtypes = [I, I, I, I, I] + [P] * 9 + [D, U64, U64] + [P] * 6 + [I]
        lib.oracle_verify_block.restype = I
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _dtype_code(dtype: str) -> int:
    return {"f32": 0, "bf16": 1}[dtype]


def _arr(a, dtype: str):
    """Contiguous float32 or bf16-bit (uint16) array, as the GPU would see it."""
    if a is None:
        return None
    want = np.float32 if dtype == "f32" else np.uint16
    a = np.ascontiguousarray(a)
    if a.dtype != want:
        raise TypeError("expected %s data for dtype %s, got %s" % (want, dtype, a.dtype))
    return a


def philox4x32_10(ctr: Sequence[int], key: Sequence[int]) -> np.ndarray:
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    _load().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def uniform(seed: int, offset: int, b: int, k: int, v: int) -> float:
    return _load().oracle_uniform(seed, offset, b, k, v)


def gumbel(seed: int, offset: int, b: int, k: int, v: int) -> float:
    return _load().oracle_gumbel(seed, offset, b, k, v)


def draft_block(inp, seed: int = 0, offset: int = 0, forced_prev=None,
                temperature=None, block_ids=None, nthreads: int = 0) -> dict:
    """Sample gamma tokens for each of the B blocks of `inp` (a synth.Inputs).
    `block_ids` gives each block's index for the noise counter (default 0..B-1)."""
    B, g = inp.B, inp.gamma
    dt = inp.dtype
    temp = np.ascontiguousarray(inp.temperature if temperature is None else temperature,
                                dtype=np.float32)
    anchor = np.ascontiguousarray(inp.anchor, dtype=np.int32)
    fp = None if forced_prev is None else np.ascontiguousarray(forced_prev, dtype=np.int32)
    ids = None if block_ids is None else np.ascontiguousarray(block_ids, dtype=np.int32)
    out = dict(
        tokens=np.zeros((B, g), np.int32), logp=np.zeros((B, g)), conf=np.zeros((B, g)),
        surv=np.zeros((B, g)), gap=np.zeros((B, g)), second=np.zeros((B, g), np.int32),
    )
    rc = _load().oracle_draft_block(
        inp.V, inp.r, inp.d, g, B, _dtype_code(dt), 1 if inp.head == "rnn" else 0,
        _ptr(_arr(inp.U, dt)), _ptr(_arr(inp.h, dt)), _ptr(anchor),
        _ptr(_arr(inp.W1, dt)), _ptr(_arr(inp.W2, dt)), _ptr(_arr(inp.w_conf, dt)),
        _ptr(_arr(inp.W_rnn, dt)), _ptr(temp), seed, offset, _ptr(fp), _ptr(ids),
        _ptr(out["tokens"]), _ptr(out["logp"]), _ptr(out["conf"]), _ptr(out["surv"]),
        _ptr(out["gap"]), _ptr(out["second"]), nthreads)
    if rc != 0:
        raise ValueError("oracle_draft_block rejected its input (rc=%d)" % rc)
    return out


def block_logprob(inp, blocks, temperature=None, nthreads: int = 0) -> np.ndarray:
    """Eq 4 log-probability of each given block `blocks` [B, gamma]."""
    dt = inp.dtype
    temp = np.ascontiguousarray(inp.temperature if temperature is None else temperature,
                                dtype=np.float32)
    blk = np.ascontiguousarray(blocks, dtype=np.int32)
    out = np.zeros(inp.B)
    rc = _load().oracle_block_logprob(
        inp.V, inp.r, inp.d, inp.gamma, inp.B, _dtype_code(dt), 1 if inp.head == "rnn" else 0,
        _ptr(_arr(inp.U, dt)), _ptr(_arr(inp.h, dt)),
        _ptr(np.ascontiguousarray(inp.anchor, np.int32)),
        _ptr(_arr(inp.W1, dt)), _ptr(_arr(inp.W2, dt)), _ptr(_arr(inp.W_rnn, dt)),
        _ptr(temp), _ptr(blk), _ptr(out), nthreads)
    if rc != 0:
        raise ValueError("oracle_block_logprob rejected its input (rc=%d)" % rc)
    return out


def position_weights(gamma: int) -> np.ndarray:
    """w_k = exp(-(k-1)/gamma), k = 1..gamma (the DSpark loss weights)."""
    return np.exp(-np.arange(gamma, dtype=np.float64) / gamma)


def block_loss(inp, alpha=(0.1, 0.9, 1.0), pos_weight=None, rows=None, cols=None,
               want_dZ: bool = True, want_dW2: bool = True, nthreads: int = 0) -> dict:
    """Teacher-forced loss over the N = inp.B blocks of `inp` (needs target, labels).
    `rows` restricts the per-row outputs to those rows; `cols` returns dZ and
    dW2 only at those vocabulary columns ([rows, len(cols)], [r, len(cols)])."""
    N, g, V = inp.B, inp.gamma, inp.V
    dt = inp.dtype
    a = np.ascontiguousarray(alpha, dtype=np.float64)
    pw = position_weights(g) if pos_weight is None else np.ascontiguousarray(pos_weight, np.float64)
    rws = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    cls = None if cols is None else np.ascontiguousarray(cols, dtype=np.int32)
    count = N * g if rws is None else len(rws)
    W = V if cls is None else len(cls)
    out = dict(loss4=np.zeros(4), c_star=np.zeros(count), conf=np.zeros(count),
               dA=np.zeros(count), ce=np.zeros(count), tv=np.zeros(count), bce=np.zeros(count))
    out["dZ"] = np.zeros((count, W)) if want_dZ else None
    out["dW2"] = np.zeros((inp.r, W)) if (want_dW2 and rws is None) else None
    rc = _load().oracle_block_loss(
        V, inp.r, inp.d, g, N, _dtype_code(dt),
        _ptr(_arr(inp.U, dt)), _ptr(_arr(inp.target, dt)), _ptr(_arr(inp.h, dt)),
        _ptr(np.ascontiguousarray(inp.anchor, np.int32)),
        _ptr(np.ascontiguousarray(inp.labels, np.int32)),
        _ptr(_arr(inp.W1, dt)), _ptr(_arr(inp.W2, dt)), _ptr(_arr(inp.w_conf, dt)),
        _ptr(a), _ptr(pw), _ptr(rws), 0 if rws is None else len(rws),
        _ptr(cls), 0 if cls is None else len(cls),
        _ptr(out["loss4"]), _ptr(out["c_star"]), _ptr(out["conf"]), _ptr(out["dA"]),
        _ptr(out["ce"]), _ptr(out["tv"]), _ptr(out["bce"]),
        _ptr(out["dZ"]), _ptr(out["dW2"]), nthreads)
    if rc != 0:
        raise ValueError("oracle_block_loss rejected its input (rc=%d)" % rc)
    return out


def block_loss_backward(inp, dZ, dA, want_dW1: bool = True, want_dw: bool = True,
                        want_dh: bool = True, nthreads: int = 0) -> dict:
    """dW1, dw_conf, dh of the teacher-forced objective from given dZ [R, V]
    and dA [R] (the loss's gradients w.r.t. the draft logits and the
    confidence logits), float64.  dZ may be None when dW1 is not wanted."""
    N, g, V, r, d = inp.B, inp.gamma, inp.V, inp.r, inp.d
    dt = inp.dtype
    R = N * g
    if dZ is not None:
        dZ = np.ascontiguousarray(np.asarray(dZ, np.float64).reshape(R, V))
    elif want_dW1:
        raise ValueError("dW1 needs dZ")
    dA = np.ascontiguousarray(np.asarray(dA, np.float64).reshape(R))
    out = dict(dW1=np.zeros((V, r)) if want_dW1 else None,
               dw=np.zeros(d + r) if want_dw else None,
               dh=np.zeros((R, d)) if want_dh else None)
    rc = _load().oracle_block_loss_backward(
        V, r, d, g, N, _dtype_code(dt), _ptr(_arr(inp.h, dt)),
        _ptr(np.ascontiguousarray(inp.anchor, np.int32)),
        _ptr(np.ascontiguousarray(inp.labels, np.int32)),
        _ptr(_arr(inp.W1, dt)), _ptr(_arr(inp.W2, dt)), _ptr(_arr(inp.w_conf, dt)),
        _ptr(dZ), _ptr(dA), _ptr(out["dW1"]), _ptr(out["dw"]), _ptr(out["dh"]), nthreads)
    if rc != 0:
        raise ValueError("oracle_block_loss_backward rejected its input (rc=%d)" % rc)
    return out


def verify_uniform(seed: int, offset: int, b: int, k: int) -> float:
    return _load().oracle_verify_uniform(seed, offset, b, k)


def verify_gumbel(seed: int, offset: int, b: int, j: int, v: int) -> float:
    return _load().oracle_verify_gumbel(seed, offset, b, j, v)


def verify_block(inp, tokens, logp, surv, target, tau: float, seed: int = 0, offset: int = 0,
                 temperature=None, nthreads: int = 0) -> dict:
    """Trim by survival >= tau, accept/reject the drafted `tokens` [B, gamma]
    against `target` logits [B, gamma + 1, V] (stored like inp.U), then draw
    the next token (see oracle_verify_block)."""
    B, g, V = inp.B, inp.gamma, inp.V
    dt = inp.dtype
    temp = np.ascontiguousarray(inp.temperature if temperature is None else temperature,
                                dtype=np.float32)
    out = dict(keep=np.zeros(B, np.int32), accept=np.zeros(B, np.int32),
               next=np.zeros(B, np.int32), margin=np.zeros(B), gap=np.zeros(B),
               accept_prob=np.zeros((B, g)))
    rc = _load().oracle_verify_block(
        V, inp.r, g, B, _dtype_code(dt), _ptr(_arr(inp.U, dt)),
        _ptr(np.ascontiguousarray(inp.anchor, np.int32)), _ptr(_arr(inp.W1, dt)),
        _ptr(_arr(inp.W2, dt)), _ptr(np.ascontiguousarray(tokens, np.int32)),
        _ptr(np.ascontiguousarray(logp, np.float64)), _ptr(np.ascontiguousarray(surv, np.float64)),
        _ptr(temp), _ptr(_arr(target, dt)), float(tau), seed, offset,
        _ptr(out["keep"]), _ptr(out["accept"]), _ptr(out["next"]), _ptr(out["margin"]),
        _ptr(out["gap"]), _ptr(out["accept_prob"]), nthreads)
    if rc != 0:
        raise ValueError("oracle_verify_block rejected its input (rc=%d)" % rc)
    return out
