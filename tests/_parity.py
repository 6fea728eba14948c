"""Comparison rules between the HIP path and the CPU oracle.

Tolerances (fixed for this method):
  tokens   exact, except where the oracle's two largest perturbed logits are
           closer than 1e-5 (but not equal) and the GPU chose the runner-up;
           at an exact tie (gap 0) the lowest index, which is the oracle's
           token, is required;
  logp     |delta log p| <= 2e-3, i.e. 2e-3 relative on the probability;
  conf, survival, c*, losses   relative 2e-3;
  dlogits  per-row relative L2 <= 2e-3; dW2 per-column and Frobenius
           relative L2 <= 2e-3.
The oracle is conditioned on the GPU's own previous tokens, so one permitted
near-tie does not cascade into later positions.
"""
from __future__ import annotations

import sys

import numpy as np

import oracle

TIE = 1e-5
RTOL = 2e-3


def note(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def check_draft(inp, gpu: dict, seed: int, offset: int, block_ids=None, label: str = "") -> dict:
    """gpu: numpy tokens/logp/conf/survival for the blocks of `inp`."""
    tok = np.asarray(gpu["tokens"])
    ora = oracle.draft_block(inp, seed=seed, offset=offset, forced_prev=tok, block_ids=block_ids)
    eq = tok == ora["tokens"]
    tie_ok = (~eq) & (ora["gap"] > 0) & (ora["gap"] < TIE) & (tok == ora["second"])
    bad = ~(eq | tie_ok)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        rows = [(int(b), int(k), int(tok[b, k]), int(ora["tokens"][b, k]), float(ora["gap"][b, k]))
                for b, k in idx]
        raise AssertionError("%s: %d token mismatches (b, k, gpu, oracle, gap): %s"
                             % (label, int(bad.sum()), rows))
    if "logp" in gpu and gpu["logp"] is not None:
        d = np.abs(np.asarray(gpu["logp"], np.float64) - ora["logp"])[eq]
        assert d.size == 0 or d.max() <= RTOL, "%s: logp max |delta| %.3g" % (label, d.max())
    for key, okey in (("conf", "conf"), ("survival", "surv")):
        g = np.asarray(gpu[key], np.float64)
        rel = np.abs(g - ora[okey]) / np.abs(ora[okey])
        assert rel.max() <= RTOL, "%s: %s max rel err %.3g" % (label, key, rel.max())
    return dict(ties=int(tie_ok.sum()), mism=0,
                logp_err=float(np.abs(np.asarray(gpu["logp"], np.float64) - ora["logp"])[eq].max()))


def rel_l2(a, b, axis=None):
    num = np.sqrt(np.sum((np.asarray(a, np.float64) - b) ** 2, axis=axis))
    den = np.sqrt(np.sum(np.asarray(b, np.float64) ** 2, axis=axis))
    return num / np.maximum(den, 1e-300)


def bf16_round(x):
    """float64 -> float32 -> bfloat16 (nearest even) -> float64, the storage
    rounding a bf16 output applies to a float32 result."""
    import synth
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(np.asarray(x, np.float32))).astype(np.float64)


def bf16_ulp(x):
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), 1e-38)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def check_loss(inp, gpu: dict, ref: dict, rows=None, label: str = "", dz_bf16: bool = False):
    """gpu: numpy loss4 [4], c_star/conf/dconf [R], dlogits [R, V] (or the
    listed rows), dW2 [r, V] (optional); ref: oracle.block_loss output over
    the same rows (all rows when `rows` is None).

    bf16 dlogits: storing to bf16 alone moves an element by up to 2^-8 of
    itself, so the reference is the oracle's dZ rounded the same way; every
    element must be within one bf16 ulp of it, rows within 2e-3 relative L2,
    and dW2 (computed from the stored dlogits) is compared with E^T times
    that rounded dZ."""
    R = inp.B * inp.gamma
    sel = np.arange(R) if rows is None else np.asarray(rows)
    cs_g = np.asarray(gpu["c_star"], np.float64).reshape(-1)[sel]
    rel = np.abs(cs_g - ref["c_star"]) / np.maximum(np.abs(ref["c_star"]), 1e-6)
    assert rel.max() <= RTOL, "%s: c* max rel err %.3g" % (label, rel.max())
    if gpu.get("conf") is not None:
        c_g = np.asarray(gpu["conf"], np.float64).reshape(-1)[sel]
        rel = np.abs(c_g - ref["conf"]) / ref["conf"]
        assert rel.max() <= RTOL, "%s: conf max rel err %.3g" % (label, rel.max())
    if gpu.get("dconf") is not None:
        d_g = np.asarray(gpu["dconf"], np.float64).reshape(-1)[sel]
        scale = np.abs(ref["dA"]).max()
        err = np.abs(d_g - ref["dA"]).max() / max(scale, 1e-30)
        assert err <= RTOL, "%s: dconf max err / max |ref| %.3g" % (label, err)
    if rows is None:
        l4 = np.asarray(gpu["loss4"], np.float64)
        rel = np.abs(l4 - ref["loss4"]) / np.abs(ref["loss4"])
        assert rel.max() <= RTOL, "%s: loss4 rel err %s" % (label, rel)
    ref_dz = ref.get("dZ")
    if ref_dz is not None and dz_bf16:
        ref_dz = bf16_round(ref_dz)
    if gpu.get("dlogits") is not None and ref_dz is not None:
        dz = np.asarray(gpu["dlogits"], np.float64).reshape(len(sel), -1)
        e = rel_l2(dz, ref_dz, axis=1)
        assert e.max() <= RTOL, "%s: dlogits max per-row rel L2 %.3g" % (label, e.max())
        if dz_bf16:
            off = np.abs(dz - ref_dz) / bf16_ulp(ref_dz)
            assert off.max() <= 1.0 + 1e-9, "%s: dlogits %.3g bf16 ulp off" % (label, off.max())
    ref_dw2 = ref.get("dW2")
    if ref_dw2 is not None and dz_bf16 and gpu.get("dlogits") is not None and rows is None:
        prev = np.concatenate([inp.anchor[:, None], inp.labels[:, :-1]], axis=1).reshape(-1)
        E = inp.as_f32(inp.W1)[prev].astype(np.float64)
        ref_dw2 = E.T @ np.asarray(gpu["dlogits"], np.float64).reshape(len(sel), -1)
    if gpu.get("dW2") is not None and ref_dw2 is not None:
        w = np.asarray(gpu["dW2"], np.float64)
        ec = rel_l2(w, ref_dw2, axis=0)
        ef = rel_l2(w, ref_dw2)
        assert ec.max() <= RTOL and ef <= RTOL, \
            "%s: dW2 per-column %.3g, Frobenius %.3g" % (label, ec.max(), ef)
