"""Comparison rules between the HIP path and the CPU oracle.

Tolerances (fixed for this method):
  tokens   exact, except where the oracle's two largest perturbed logits are
           closer than 1e-5 and the GPU chose the runner-up;
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
    tie_ok = (~eq) & (ora["gap"] < TIE) & (tok == ora["second"])
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
