"""torch-facing wrappers over the C ABI: shape inference, output and
workspace allocation, then one call into libdspark.so.  All arithmetic runs
in the HIP library; torch only provides device memory and the stream."""
from __future__ import annotations

from typing import Optional

import torch

from . import binding as _b

_DTYPES = {torch.bfloat16: "bf16", torch.float32: "f32"}


def _dtype_of(t: torch.Tensor) -> str:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError("tensors must be bfloat16 or float32, got %s" % t.dtype) from None


def draft_dims(U, h, W1, W_rnn=None) -> _b.dspark_dims:
    B, gamma, V = U.shape
    return _b.make_dims(V, W1.shape[1], h.shape[-1], gamma, B, _dtype_of(U),
                        "rnn" if W_rnn is not None else "markov")


def workspace(dims: _b.dspark_dims, which: int, device) -> torch.Tensor:
    n = _b.dspark_workspace_size(dims, which)
    if n == 0:
        raise _b.DsparkError(_b.DSPARK_EINVAL, _b.dspark_last_error())
    return torch.empty(n, dtype=torch.uint8, device=device)


def draft_block(U, h, anchor, W1, W2, w_conf, temperature, *, W_rnn=None, seed: int = 0,
                offset: int = 0, out: Optional[dict] = None, ws: Optional[torch.Tensor] = None,
                stream=None) -> dict:
    """Draft gamma tokens for each of the B blocks (see dspark_draft_block)."""
    dims = draft_dims(U, h, W1, W_rnn)
    dev = U.device
    B, gamma = dims.B, dims.gamma
    if out is None:
        out = dict(tokens=torch.empty((B, gamma), dtype=torch.int32, device=dev),
                   logp=torch.empty((B, gamma), dtype=torch.float32, device=dev),
                   conf=torch.empty((B, gamma), dtype=torch.float32, device=dev),
                   survival=torch.empty((B, gamma), dtype=torch.float32, device=dev))
    if ws is None:
        ws = workspace(dims, _b.DSPARK_CALL_DRAFT, dev)
    _b.dspark_draft_block(dims, U, h, anchor, W1, W2, w_conf, W_rnn, temperature, seed, offset,
                          out["tokens"], out.get("logp"), out["conf"], out["survival"], ws,
                          stream=stream)
    out["_ws"] = ws
    out["_dims"] = dims
    return out


def block_loss(U, T_logits, h, anchor, labels, W1, W2, w_conf, *, alpha=None, pos_weight=None,
               dlogits_dtype: Optional[str] = "f32", want_dW2: bool = True,
               ws: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Teacher-forced loss, dlogits and dW2 (see dspark_block_loss)."""
    N, gamma, V = U.shape
    dims = _b.make_dims(V, W1.shape[1], h.shape[-1], gamma, N, _dtype_of(U), "markov")
    dev = U.device
    out = dict(loss4=torch.empty(4, dtype=torch.float32, device=dev),
               c_star=torch.empty((N, gamma), dtype=torch.float32, device=dev),
               conf=torch.empty((N, gamma), dtype=torch.float32, device=dev),
               dconf_logit=torch.empty((N, gamma), dtype=torch.float32, device=dev))
    out["dlogits"] = None
    if dlogits_dtype is not None:
        td = torch.float32 if dlogits_dtype == "f32" else torch.bfloat16
        out["dlogits"] = torch.empty((N, gamma, V), dtype=td, device=dev)
    out["dW2"] = torch.empty((W1.shape[1], V), dtype=torch.float32, device=dev) if want_dW2 else None
    if ws is None:
        ws = workspace(dims, _b.DSPARK_CALL_LOSS, dev)
    _b.dspark_block_loss(dims, U, T_logits, h, anchor, labels, W1, W2, w_conf, alpha, pos_weight,
                         out["loss4"], out["c_star"], out["conf"], out["dlogits"],
                         dlogits_dtype or "f32", out["dW2"], out["dconf_logit"], ws, stream=stream)
    out["_ws"] = ws
    out["_dims"] = dims
    return out


def block_loss_backward(dlogits, dconf_logit, h, anchor, labels, W1, W2, w_conf, *,
                        want_dW1: bool = True, want_dw_conf: bool = True, want_dh: bool = True,
                        ws: Optional[torch.Tensor] = None, stream=None) -> dict:
    """dW1, dw_conf and dh from the loss call's dlogits and dconf_logit
    (see dspark_block_loss_backward)."""
    N, gamma, d = h.shape
    V, r = W1.shape
    dims = _b.make_dims(V, r, d, gamma, N, _dtype_of(W1), "markov")
    dev = W1.device
    out = dict(
        dW1=torch.empty((V, r), dtype=torch.float32, device=dev) if want_dW1 else None,
        dw_conf=torch.empty(d + r, dtype=torch.float32, device=dev) if want_dw_conf else None,
        dh=torch.empty((N, gamma, d), dtype=torch.float32, device=dev) if want_dh else None)
    if ws is None:
        ws = workspace(dims, _b.DSPARK_CALL_LOSS_BACKWARD, dev)
    dz_dtype = "f32" if dlogits is None else _dtype_of(dlogits)
    _b.dspark_block_loss_backward(dims, dlogits, dz_dtype, dconf_logit, h, anchor, labels, W1, W2,
                                  w_conf, out["dW1"], out["dw_conf"], out["dh"], ws, stream=stream)
    out["_ws"] = ws
    out["_dims"] = dims
    return out


def verify_block(U, anchor, W1, W2, T_logits, tokens, logp, survival, temperature, *,
                 threshold: float = 0.0, seed: int = 0, offset: int = 0, want_accept_prob=True,
                 ws: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Trim, accept/reject and the next token for drafted blocks (see
    dspark_verify_block)."""
    B, gamma, V = U.shape
    dims = _b.make_dims(V, W1.shape[1], 1, gamma, B, _dtype_of(U), "markov")
    dev = U.device
    out = dict(n_keep=torch.empty(B, dtype=torch.int32, device=dev),
               n_accept=torch.empty(B, dtype=torch.int32, device=dev),
               next_token=torch.empty(B, dtype=torch.int32, device=dev),
               accept_prob=torch.empty((B, gamma), dtype=torch.float32, device=dev)
               if want_accept_prob else None)
    if ws is None:
        ws = workspace(dims, _b.DSPARK_CALL_VERIFY, dev)
    _b.dspark_verify_block(dims, U, anchor, W1, W2, T_logits, tokens, logp, survival, temperature,
                           threshold, seed, offset, out["n_keep"], out["n_accept"],
                           out["next_token"], out["accept_prob"], ws, stream=stream)
    out["_ws"] = ws
    out["_dims"] = dims
    return out
