#!/usr/bin/env python3
"""Throughput of DSpark block drafting on one MI355X.

A step is one dspark_draft_block call over the Qwen3-4B-shaped workload:
B = 32 anchors, gamma = 7 positions, V = 151936, Markov rank r = 256, hidden
d = 2560, bf16 weights and base logits, temperature 1 (Gumbel-max sampling).
Inputs are seeded synthetic tensors resident in HBM before timing starts.
Each step uses a new noise offset (offset = step index).

Prints one JSON line: drafted tokens/s over the K timed steps, the roofline
of the dominant kernel (the single-launch drafting kernel, or the V-streaming
step kernel of the per-step driver, timed with HIP events on the library's
stream during the timed region) and the CPU oracle's rate on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "drafted block-tokens/s (V=151936, r=256, γ=7) + % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
WORKLOAD_CFG = 2
COUNTERS = os.path.join(ROOT, "profiles", "draft_persistent_counters.json")
KERNEL_SOURCES = [os.path.join(ROOT, "semi_autoregressive_draft_markov_amd", "csrc", f)
                  for f in ("draft.hip", "draft_persistent.hip", "mfma_tile.h", "device_common.h",
                            "internal.h")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from committed rocprofv3 counter runs
    (FETCH_SIZE + WRITE_SIZE, scaled by a copy-kernel calibration), or None
    if absent, taken on another kernel, or on a different kernel source."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_hash") != kernel_source_hash() or c.get("kernel") != kernel:
        return None
    return c.get("bytes_per_launch")


def cpu_threads() -> int:
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        n = min(n, int(env))
    return max(1, n)


def cpu_baseline(inp, seconds: float):
    """The CPU oracle on the same inputs, repeated whole-batch calls until
    `seconds` of wall time have passed (at least one)."""
    import oracle
    threads = cpu_threads()
    oracle.draft_block(synth_subset(inp, [0]), nthreads=1)  # load the library
    t0 = time.perf_counter()
    calls = 0
    while True:
        oracle.draft_block(inp, seed=0, offset=calls, nthreads=threads)
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    toks = calls * inp.B * inp.gamma
    return dict(value=toks / el, unit="tokens/s", cores=threads, kind="oracle",
                sample="%d whole-batch call(s) of the workload (%d blocks x %d positions), "
                       "%.1f s wall, fp64 C oracle, OpenMP over blocks"
                       % (calls, inp.B, inp.gamma, el))


def copy_calibration() -> int:
    """A plain 1 GiB device-to-device copy, five times: reads and writes
    exactly 2^30 bytes per launch, the yardstick for the FETCH_SIZE and
    WRITE_SIZE counters of the stream kernel."""
    import torch
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}), flush=True)
    return 0


def bench_loss(args) -> int:
    """Teacher-forced loss over the Qwen3-8B-shaped workload: 1024 blocks x
    7 positions = 7168 rows, V = 151936, r = 256, d = 4096, bf16 inputs,
    bf16 dlogits and float32 dW2.  A step is one dspark_block_loss call."""
    import torch

    import synth
    from semi_autoregressive_draft_markov_amd import binding, ops

    binding.load()
    dev = torch.device("cuda:0")
    inp = synth.config_inputs(3)
    t = synth.to_torch(inp, dev)
    R, V, r = inp.B * inp.gamma, inp.V, inp.r
    out = ops.block_loss(t["U"], t["target"], t["h"], t["anchor"], t["labels"], t["W1"], t["W2"],
                         t["w_conf"], dlogits_dtype="bf16")
    dims, ws = out["_dims"], out["_ws"]

    def step():
        binding.dspark_block_loss(dims, t["U"], t["target"], t["h"], t["anchor"], t["labels"],
                                  t["W1"], t["W2"], t["w_conf"], None, None, out["loss4"],
                                  out["c_star"], out["conf"], out["dlogits"], "bf16", out["dW2"],
                                  out["dconf_logit"], ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    binding.dspark_profile_enable(True)
    binding.dspark_profile_read()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    pass_ms, launches = binding.dspark_profile_read()
    binding.dspark_profile_enable(False)
    # the three passes' own inputs and outputs: passes 1 and 2 read U and T,
    # pass 3 reads U and writes bf16 dlogits (its sign bits from pass 2 are
    # an implementation detail and not counted)
    alg_bytes = 2 * (2 * R * V * 2) + 2 * R * V * 2
    pass_s = pass_ms * 1e-3 / args.steps
    line = {
        "metric": "teacher-forced rows/s (V=151936, r=256, γ=7, 7168 rows)",
        "value": round(R * args.steps / el, 1), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(el * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3-8b-shaped teacher-forced loss", "V": V, "r": r,
                   "d": inp.d, "gamma": inp.gamma, "N": inp.B, "dlogits": "bf16"},
        "roofline": {"bound": "hbm", "achieved": round(alg_bytes / pass_s / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(alg_bytes / pass_s / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "k_loss_mfma passes 1-3", "passes_ms": round(pass_ms / args.steps, 4)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_backward(args) -> int:
    """Backward past the logits over the Qwen3-8B-shaped workload (7168 rows,
    V = 151936, r = 256, d = 4096): one dspark_block_loss call makes bf16
    dlogits and dconf_logit, then a step is one dspark_block_loss_backward
    call (dW1, dw_conf, dh).  Roofline of its dZ W2^T kernel: the dZ stream
    plus one pass over W2 per launch, against HBM."""
    import torch

    import synth
    from semi_autoregressive_draft_markov_amd import binding, ops

    binding.load()
    dev = torch.device("cuda:0")
    inp = synth.config_inputs(3)
    t = synth.to_torch(inp, dev)
    R, V, r, d = inp.B * inp.gamma, inp.V, inp.r, inp.d
    lo = ops.block_loss(t["U"], t["target"], t["h"], t["anchor"], t["labels"], t["W1"], t["W2"],
                        t["w_conf"], dlogits_dtype="bf16", want_dW2=False)
    out = ops.block_loss_backward(lo["dlogits"], lo["dconf_logit"], t["h"], t["anchor"],
                                  t["labels"], t["W1"], t["W2"], t["w_conf"])
    dims, ws = out["_dims"], out["_ws"]
    del t["U"], t["target"]

    def step():
        binding.dspark_block_loss_backward(dims, lo["dlogits"], "bf16", lo["dconf_logit"], t["h"],
                                           t["anchor"], t["labels"], t["W1"], t["W2"],
                                           t["w_conf"], out["dW1"], out["dw_conf"], out["dh"], ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    binding.dspark_profile_enable(True)
    binding.dspark_profile_read()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    de_ms, launches = binding.dspark_profile_read()
    binding.dspark_profile_enable(False)
    de_s = de_ms * 1e-3 / max(launches, 1)
    alg_bytes = R * V * 2 + r * V * 2
    flops = 2.0 * R * V * r
    line = {
        "metric": "teacher-forced rows/s through the backward past the logits (V=151936, r=256, "
                  "d=4096, 7168 rows)",
        "value": round(R * args.steps / el, 1), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(el * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3-8b-shaped backward past the logits", "V": V, "r": r,
                   "d": d, "gamma": inp.gamma, "N": inp.B, "dlogits": "bf16"},
        "roofline": {"bound": "hbm", "achieved": round(alg_bytes / de_s / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(alg_bytes / de_s / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "k_de_mfma<8, 2, false>", "kernel_ms": round(de_s * 1e3, 4),
                     "mfma_tflops": round(flops / de_s / 1e12, 1)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_verify(args) -> int:
    """Verification of Qwen3-4B-shaped drafted blocks (B = 32, gamma = 7,
    V = 151936, r = 256, bf16): one dspark_draft_block call drafts the
    blocks, synthetic target logits [B, gamma + 1, V] (the base logits plus
    N(0, 0.3^2) at the drafted positions) stand in for the target model;
    a step is one dspark_verify_block call (threshold 0.25).  Roofline of its
    draft-row kernel: W2 once, the U rows of the residual positions and the
    float32 draft rows it writes."""
    import numpy as np
    import torch

    import synth
    from semi_autoregressive_draft_markov_amd import binding, ops

    binding.load()
    dev = torch.device("cuda:0")
    inp = synth.config_inputs(WORKLOAD_CFG)
    t = synth.to_torch(inp, dev)
    B, gamma, V, r = inp.B, inp.gamma, inp.V, inp.r
    d = ops.draft_block(t["U"], t["h"], t["anchor"], t["W1"], t["W2"], t["w_conf"], t["temperature"])
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    tgt = torch.empty((B, gamma + 1, V), dtype=torch.bfloat16, device=dev)
    tgt[:, :gamma] = (t["U"].float() + 0.3 * torch.randn((B, gamma, V), generator=g, device=dev)).bfloat16()
    tgt[:, gamma] = (2.0 * torch.randn((B, V), generator=g, device=dev)).bfloat16()
    out = ops.verify_block(t["U"], t["anchor"], t["W1"], t["W2"], tgt, d["tokens"], d["logp"],
                           d["survival"], t["temperature"], threshold=0.25)
    dims, ws = out["_dims"], out["_ws"]

    def step(i):
        binding.dspark_verify_block(dims, t["U"], t["anchor"], t["W1"], t["W2"], tgt, d["tokens"],
                                    d["logp"], d["survival"], t["temperature"], 0.25, 0, i,
                                    out["n_keep"], out["n_accept"], out["next_token"],
                                    out["accept_prob"], ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    binding.dspark_profile_enable(True)
    binding.dspark_profile_read()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    k_ms, launches = binding.dspark_profile_read()
    binding.dspark_profile_enable(False)
    k_s = k_ms * 1e-3 / max(launches, 1)
    alg_bytes = r * V * 2 + B * V * 2 + B * V * 4
    acc = out["n_accept"].float().mean().item()
    line = {
        "metric": "verified blocks/s (V=151936, r=256, γ=7, B=32)",
        "value": round(B * args.steps / el, 1), "unit": "blocks/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(el * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3-4b-shaped verification of drafted blocks", "V": V, "r": r,
                   "gamma": gamma, "B": B, "threshold": 0.25,
                   "mean_accepted": round(acc, 3)},
        "roofline": {"bound": "hbm", "achieved": round(alg_bytes / k_s / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(alg_bytes / k_s / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "k_v_bias_mfma<8>", "kernel_us": round(k_s * 1e6, 2)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    return 0


def synth_subset(inp, idx):
    import synth
    return synth.subset(inp, idx)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall time of the CPU oracle sample (0 skips it)")
    ap.add_argument("--workload", default="qwen3-4b",
                    choices=["qwen3-4b", "qwen3-14b", "gemma4-rnn", "qwen3-8b-loss",
                             "qwen3-8b-backward", "qwen3-4b-verify"],
                    help="qwen3-4b (default) is the reported workload; the others are "
                         "extra measurements of the same kernels at the other shapes")
    ap.add_argument("--flush", action="store_true",
                    help="write a 1 GiB buffer before every timed drafting call (untimed) so that "
                         "W2 and U come from HBM, not from the 256 MB memory-side cache; the "
                         "value is then B*gamma*steps over the summed per-call event times")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="instead of the benchmark, run a plain device copy of 1 GiB "
                         "(reference for HBM byte counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        return copy_calibration()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the drafting path has no cross-GPU work "
              "(blocks are independent); run it with --gpus 1", file=sys.stderr)
        return 2

    if args.workload == "qwen3-8b-loss":
        return bench_loss(args)
    if args.workload == "qwen3-8b-backward":
        return bench_backward(args)
    if args.workload == "qwen3-4b-verify":
        return bench_verify(args)

    import numpy as np
    import torch

    import synth
    from semi_autoregressive_draft_markov_amd import binding, ops

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    binding.load()
    dev = torch.device("cuda:0")
    cfg = {"qwen3-4b": 2, "qwen3-14b": 4, "gemma4-rnn": 5}[args.workload]
    inp = synth.config_inputs(cfg)
    t = synth.to_torch(inp, dev)
    B, gamma, V, r, d = inp.B, inp.gamma, inp.V, inp.r, inp.d
    dims = ops.draft_dims(t["U"], t["h"], t["W1"], t["W_rnn"])
    ws = ops.workspace(dims, binding.DSPARK_CALL_DRAFT, dev)
    out = dict(tokens=torch.empty((B, gamma), dtype=torch.int32, device=dev),
               logp=torch.empty((B, gamma), dtype=torch.float32, device=dev),
               conf=torch.empty((B, gamma), dtype=torch.float32, device=dev),
               survival=torch.empty((B, gamma), dtype=torch.float32, device=dev))
    stream = torch.cuda.current_stream()

    def step(i):
        binding.dspark_draft_block(dims, t["U"], t["h"], t["anchor"], t["W1"], t["W2"],
                                   t["w_conf"], t["W_rnn"], t["temperature"], 0, i, out["tokens"],
                                   out["logp"], out["conf"], out["survival"], ws, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    binding.dspark_profile_enable(True)
    binding.dspark_profile_read()
    torch.cuda.synchronize()
    if args.flush:
        scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for i in range(args.steps):
            scratch.zero_()
            evs[i][0].record(stream)
            step(args.warmup + i)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        elapsed = sum(a.elapsed_time(b) for a, b in evs) * 1e-3
    else:
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(args.warmup + i)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    kernel_ms, launches = binding.dspark_profile_read()
    binding.dspark_profile_enable(False)
    per_call = launches // args.steps
    assert per_call * args.steps == launches and per_call in (1, gamma), (launches, args.steps)
    tokens = out["tokens"].cpu().numpy()
    assert np.all((tokens >= 0) & (tokens < V)), "bad tokens"

    ms_per_step = elapsed * 1e3 / args.steps
    value = B * gamma * args.steps / elapsed
    avg_kernel_s = kernel_ms * 1e-3 / launches
    kname = binding.dspark_draft_kernel_name(dims)
    if per_call == 1:
        # single-launch driver: W2 is read once per call, every step's U slice once
        driver = "single-launch"
        alg_bytes = (r + gamma * B) * V * 2
    else:
        # per-step driver: every step streams all of W2 plus its slice of U
        driver = "per-step"
        alg_bytes = (r + B) * V * 2
    names = {"qwen3-4b": "qwen3-4b-shaped markov-head block sampling",
             "qwen3-14b": "qwen3-14b-shaped markov-head block sampling, half greedy",
             "gemma4-rnn": "gemma4-12b-shaped rnn-head block sampling"}
    achieved = alg_bytes / avg_kernel_s / 1e9
    traffic = measured_traffic(kname)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": names[args.workload],
                   "V": V, "r": r, "d": d, "gamma": gamma, "B": B,
                   "head": inp.head, "parallelism": "single-gpu",
                   **({"caches": "flushed before every call"} if args.flush else {})},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic if args.workload == "qwen3-4b" else None,
                     "kernel": kname, "driver": driver,
                     "kernel_us": round(avg_kernel_s * 1e6, 3),
                     "algorithmic_bytes_per_launch": alg_bytes},
    }
    if args.cpu_seconds > 0:
        line["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
