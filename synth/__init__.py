"""Seeded synthetic inputs for the DSpark sequential head.

This module only draws random tensors.  It holds none of the method's
arithmetic: no bias, softmax, sampling, confidence or loss.  Both the CPU
oracle (via the tests) and the HIP path (via the tests and the benchmark)
consume what it returns, so the two sides always see the same bytes.

Shapes and value laws follow the workloads the DSpark pages describe: the
Qwen3-4B/8B/14B and Gemma4-12B drafters (block size 7, Markov rank 256,
DSpark paper section 4.1 as transcribed on the dormouse verification note,
section 1), with the distributions of the CONFIGS table below.

Layouts (all C-contiguous):
  anchor [B] int32, U [B, gamma, V], h [B, gamma, d], W1 [V, r], W2 [r, V],
  w_conf [d + r] (h part first), W_rnn [3r, 2r + d] (rows g, c, o; columns
  s, e, h), temperature [B] float32, target [B, gamma, V], labels [B, gamma].
Floating tensors are numpy float32 for dtype "f32", and numpy uint16 holding
bfloat16 bit patterns (round-to-nearest-even from float32) for dtype "bf16".
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

DTYPES = ("f32", "bf16")
HEADS = ("markov", "rnn")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def zipf_tokens(rng: np.random.Generator, n: int, V: int, s: float = 1.1) -> np.ndarray:
    """Finite Zipf law over [0, V): P(v) proportional to (v + 1)^-s, inverse CDF."""
    p = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(p)
    cdf /= cdf[-1]
    u = rng.random(n)
    return np.minimum(np.searchsorted(cdf, u, side="right"), V - 1).astype(np.int32)


@dataclasses.dataclass
class Inputs:
    V: int
    r: int
    d: int
    gamma: int
    B: int
    dtype: str
    head: str
    anchor: np.ndarray
    U: np.ndarray
    h: np.ndarray
    W1: np.ndarray
    W2: np.ndarray
    w_conf: np.ndarray
    W_rnn: Optional[np.ndarray]
    temperature: np.ndarray
    target: Optional[np.ndarray] = None
    labels: Optional[np.ndarray] = None
    name: str = ""

    def as_f32(self, a: Optional[np.ndarray]) -> Optional[np.ndarray]:
        """Exact float32 view of a floating input (widening bf16 bits)."""
        if a is None:
            return None
        return bf16_bits_to_f32(a) if self.dtype == "bf16" else a


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def make_inputs(
    *,
    V: int,
    r: int,
    d: int,
    gamma: int,
    B: int,
    dtype: str = "bf16",
    head: str = "markov",
    seed: int = 0,
    u_std: float = 3.0,
    h_std: float = 1.0,
    w1_std: float = 0.02,
    w2_std: float = 0.02,
    wconf_std: float = 0.02,
    wrnn_std: float = 0.02,
    anchors: str = "zipf",
    temperature=1.0,
    target_noise_std: Optional[float] = None,
    name: str = "",
) -> Inputs:
    """Draw one synthetic problem.

    Draw order is fixed: anchors, U, h, W1, W2, w_conf, W_rnn, target noise.
    `temperature` is a scalar or a length-B sequence (0 means greedy).
    `target_noise_std` set => also draw target logits = U + noise and labels =
    the first index of the target's maximum (training inputs).
    """
    assert dtype in DTYPES and head in HEADS
    rng = np.random.Generator(np.random.PCG64(seed))
    if anchors == "zipf":
        anchor = zipf_tokens(rng, B, V)
    elif anchors == "uniform":
        anchor = rng.integers(0, V, size=B, dtype=np.int64).astype(np.int32)
    else:
        raise ValueError(anchors)
    f32 = np.float32
    U = rng.standard_normal((B, gamma, V), dtype=f32) * f32(u_std)
    h = rng.standard_normal((B, gamma, d), dtype=f32) * f32(h_std)
    W1 = rng.standard_normal((V, r), dtype=f32) * f32(w1_std)
    W2 = rng.standard_normal((r, V), dtype=f32) * f32(w2_std)
    w_conf = rng.standard_normal((d + r,), dtype=f32) * f32(wconf_std)
    W_rnn = None
    if head == "rnn":
        W_rnn = rng.standard_normal((3 * r, 2 * r + d), dtype=f32) * f32(wrnn_std)
    temp = np.broadcast_to(np.asarray(temperature, dtype=f32), (B,)).copy()
    out = Inputs(
        V=V, r=r, d=d, gamma=gamma, B=B, dtype=dtype, head=head,
        anchor=anchor,
        U=_cast(U, dtype), h=_cast(h, dtype), W1=_cast(W1, dtype), W2=_cast(W2, dtype),
        w_conf=_cast(w_conf, dtype),
        W_rnn=None if W_rnn is None else _cast(W_rnn, dtype),
        temperature=temp, name=name,
    )
    del U
    if target_noise_std is not None:
        Uf = out.as_f32(out.U)
        noise = rng.standard_normal(Uf.shape, dtype=f32) * f32(target_noise_std)
        tgt = _cast(Uf + noise, dtype)
        del noise
        out.target = tgt
        out.labels = np.argmax(out.as_f32(tgt), axis=-1).astype(np.int32)
    return out


# The five workloads.  Each entry gives make_inputs keyword arguments.
CONFIGS = {
    1: dict(V=1024, r=32, d=64, gamma=7, B=4, dtype="f32", head="markov",
            u_std=2.0, h_std=2.0, w1_std=0.05, w2_std=0.05, wconf_std=0.05,
            anchors="uniform", temperature=1.0, target_noise_std=1.0,
            name="tiny markov block V1024 r32 d64 B4 fp32"),
    2: dict(V=151936, r=256, d=2560, gamma=7, B=32, dtype="bf16", head="markov",
            u_std=3.0, h_std=1.0, w1_std=0.02, w2_std=0.02, wconf_std=0.02,
            anchors="zipf", temperature=1.0,
            name="qwen3-4b-shaped sampling V151936 r256 d2560 B32 bf16"),
    3: dict(V=151936, r=256, d=4096, gamma=7, B=1024, dtype="bf16", head="markov",
            u_std=3.0, h_std=1.0, w1_std=0.02, w2_std=0.02, wconf_std=0.02,
            anchors="zipf", temperature=1.0, target_noise_std=1.5,
            name="qwen3-8b-shaped teacher-forced loss V151936 r256 d4096 N1024"),
    4: dict(V=151936, r=256, d=5120, gamma=7, B=256, dtype="bf16", head="markov",
            u_std=3.0, h_std=1.0, w1_std=0.02, w2_std=0.02, wconf_std=0.02,
            anchors="zipf", temperature=[1.0] * 128 + [0.0] * 128,
            name="qwen3-14b-shaped sampling V151936 r256 d5120 B256 half greedy"),
    5: dict(V=262144, r=256, d=3840, gamma=7, B=128, dtype="bf16", head="rnn",
            u_std=3.0, h_std=1.0, w1_std=0.02, w2_std=0.02, wconf_std=0.02,
            wrnn_std=0.02, anchors="zipf", temperature=1.0,
            name="gemma4-12b-shaped rnn-head sampling V262144 r256 d3840 B128"),
}


def config_inputs(cfg: int, **overrides) -> Inputs:
    """Inputs of workload `cfg` (1..5), seeded with 1000 + cfg unless overridden."""
    kw = dict(CONFIGS[cfg])
    kw.setdefault("seed", 1000 + cfg)
    kw.update(overrides)
    return make_inputs(**kw)


def to_torch(inp: Inputs, device="cuda") -> dict:
    """Copy the arrays of `inp` to `device` as torch tensors (bf16 bits are
    reinterpreted as torch.bfloat16, not converted)."""
    import torch

    def t(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    out = {name: t(getattr(inp, name)) for name in
           ("U", "h", "W1", "W2", "w_conf", "W_rnn", "target")}
    out["anchor"] = t(np.ascontiguousarray(inp.anchor, dtype=np.int32))
    out["temperature"] = t(np.ascontiguousarray(inp.temperature, dtype=np.float32))
    out["labels"] = None if inp.labels is None else t(np.ascontiguousarray(inp.labels, np.int32))
    return out


def subset(inp: Inputs, blocks) -> Inputs:
    """The same problem restricted to the listed blocks (weights shared)."""
    blocks = np.asarray(blocks)
    c = Inputs(**{f: getattr(inp, f) for f in inp.__dataclass_fields__})
    c.B = len(blocks)
    for name in ("anchor", "temperature"):
        setattr(c, name, np.ascontiguousarray(getattr(inp, name)[blocks]))
    for name in ("U", "h", "target", "labels"):
        a = getattr(inp, name)
        if a is not None:
            setattr(c, name, np.ascontiguousarray(a[blocks]))
    return c
