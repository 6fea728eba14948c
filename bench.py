#!/usr/bin/env python3
"""Throughput of DSpark block drafting on one MI355X.

A step is one dspark_draft_block call over the Qwen3-4B-shaped workload:
B = 32 anchors, gamma = 7 positions, V = 151936, Markov rank r = 256, hidden
d = 2560, bf16 weights and base logits, temperature 1 (Gumbel-max sampling).
Inputs are seeded synthetic tensors resident in HBM before timing starts.
Each step uses a new noise offset (offset = step index).

Timing: before every timed call a 1 GiB buffer is read (untimed), so that
the weights and logits come from HBM and not from the 256 MB memory-side
cache (a read leaves the caches holding clean lines; a 1 GiB write would
leave dirty ones whose write-back the timed call would pay for); each call
is bracketed by HIP events on its stream and `value` is the drafted tokens
over the summed call times.  The same calls back to back
without the flush give `warm_value` (context only).

Prints one JSON line: the throughput, the roofline of the dominant kernel
(timed live with the library's own HIP events around that kernel, in a
second pass of the same flushed calls so that those events do not add to
the value; the bound
is the roof with the largest measured fraction -- HBM bytes, matrix-core
flops, or vector-ALU instruction issue from committed rocprofv3 counters)
and the CPU oracle's rate on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "drafted block-tokens/s (V=151936, r=256, γ=7) + % of HBM/MFMA roofline"
# MI355X published peaks
HBM_PEAK_GBS = 8000.0           # HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix cores
# vector-ALU issue: 256 compute units x 4 SIMDs x 16 lanes x 2.4 GHz (a
# wave64 instruction occupies a SIMD for 4 cycles) = 39.3 T lane-ops/s
VALU_PEAK_TLANEOPS = 256 * 4 * 16 * 2.4e9 / 1e12
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
CSRC = os.path.join(ROOT, "semi_autoregressive_draft_markov_amd", "csrc")
FLUSH_BYTES = 1 << 30


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for fn in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, fn), "rb") as f:
            h.update(fn.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def counters_for(workload: str, kernels):
    """Per-launch counters summed over `kernels` (names, or prefixes ending
    in '<' for every instance of a template) of `workload`, from the
    committed rocprofv3 runs (profiles/counters.json, written by
    collect_profiles.py); None if absent or taken on other kernel sources."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_hash") != kernel_source_hash():
        return None
    ks = c.get("workloads", {}).get(workload, {}).get("kernels", {})
    names = [kernels] if isinstance(kernels, str) else list(kernels)
    hit = [e for k, e in ks.items() if any(k == n or (n.endswith("<") and k.startswith(n)) for n in names)]
    if not hit:
        return None
    out = {}
    for key in ("fetch_kib", "write_kib", "sq_insts_valu"):
        if all(e.get(key) is not None for e in hit):
            out[key] = sum(e[key] for e in hit)
    if len(hit) == 1:
        for key in ("valu_busy_pct", "mfma_util_pct", "lds_bank_conflict_per_lds_cycle", "wait_any_per_wave_cycle"):
            if key in hit[0]:
                out[key] = hit[0][key]
    cal = c.get("copy_calibration", {})
    if "fetch_kib" in out and "write_kib" in out and cal:
        fs = FLUSH_BYTES / 1024.0 / cal["fetch_kib_per_gib"]
        ws = FLUSH_BYTES / 1024.0 / cal["write_kib_per_gib"]
        out["traffic_bytes"] = round(out["fetch_kib"] * 1024 * fs + out["write_kib"] * 1024 * ws)
        out["fetch_scale"], out["write_scale"] = round(fs, 4), round(ws, 4)
    return out


def roofline(workload, kernel, kernel_s, alg_bytes, alg_flops, match=None):
    """Fractions of the three roofs for one launch of `kernel` (or of the
    kernels `match` names, summed) taking `kernel_s` seconds; the bound is
    the largest.  The vector-ALU fraction needs the committed SQ_INSTS_VALU
    count of the same build."""
    c = counters_for(workload, match or kernel)
    fr = {"hbm": alg_bytes / kernel_s / 1e9 / HBM_PEAK_GBS,
          "mfma": alg_flops / kernel_s / 1e12 / MFMA_BF16_PEAK_TFLOPS}
    achieved = {"hbm": alg_bytes / kernel_s / 1e9, "mfma": alg_flops / kernel_s / 1e12}
    if c and "sq_insts_valu" in c:
        lane_ops = c["sq_insts_valu"] * 64.0
        achieved["alu"] = lane_ops / kernel_s / 1e12
        fr["alu"] = achieved["alu"] / VALU_PEAK_TLANEOPS
    bound = max(fr, key=fr.get)
    peak = {"hbm": HBM_PEAK_GBS, "mfma": MFMA_BF16_PEAK_TFLOPS, "alu": VALU_PEAK_TLANEOPS}[bound]
    unit = {"hbm": "GB/s", "mfma": "TFLOP/s", "alu": "Tlane-op/s"}[bound]
    line = {"bound": bound, "achieved": round(achieved[bound], 2), "peak": round(peak, 2), "unit": unit,
            "frac": round(fr[bound], 4),
            "traffic": c.get("traffic_bytes") if c else None,
            "kernel": kernel, "kernel_us": round(kernel_s * 1e6, 3),
            "algorithmic_bytes_per_launch": int(alg_bytes),
            "algorithmic_flops_per_launch": int(alg_flops),
            "fractions": {k: round(v, 4) for k, v in fr.items()}}
    if c:
        for k in ("valu_busy_pct", "mfma_util_pct", "lds_bank_conflict_per_lds_cycle", "wait_any_per_wave_cycle"):
            if k in c:
                line[k] = c[k]
    else:
        line["counters"] = "none for these kernel sources (profiles/counters.json was taken on other sources)"
    return line


def host_info() -> dict:
    nproc = os.cpu_count()
    model = ""
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    if not model:
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        model = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
    return {"nproc": nproc, "cpu_model": model}


def cpu_threads() -> int:
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        n = min(n, int(env))
    return max(1, n)


def timed_repeats(fn, seconds: float):
    """Call fn() until `seconds` of wall time have passed (at least once);
    returns (calls, elapsed)."""
    t0 = time.perf_counter()
    calls = 0
    while True:
        fn(calls)
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return calls, el


def cpu_result(value, unit, sample, threads):
    return dict(value=value, unit=unit, cores=threads, kind="oracle", sample=sample, **host_info())


def cpu_baseline_draft(inp, seconds: float):
    """The CPU oracle on the same inputs: whole-batch calls for `seconds`."""
    import oracle
    import synth
    threads = cpu_threads()
    oracle.draft_block(synth.subset(inp, [0]), nthreads=1)  # load the library
    calls, el = timed_repeats(lambda i: oracle.draft_block(inp, seed=0, offset=i, nthreads=threads),
                              seconds)
    toks = calls * inp.B * inp.gamma
    return cpu_result(toks / el, "tokens/s",
                      "%d whole-batch call(s) of the workload (%d blocks x %d positions), %.1f s wall, "
                      "fp64 C oracle, OpenMP over blocks" % (calls, inp.B, inp.gamma, el), threads)


def cpu_baseline_loss(inp, seconds: float, blocks: int = 16):
    """The oracle's teacher-forced loss with dZ and dW2 on the first `blocks`
    blocks of the workload (the same per-row work as the full call)."""
    import numpy as np
    import oracle
    import synth
    threads = cpu_threads()
    sub = synth.subset(inp, np.arange(blocks))
    rows = blocks * inp.gamma
    calls, el = timed_repeats(lambda i: oracle.block_loss(sub, nthreads=threads), seconds)
    return cpu_result(calls * rows / el, "rows/s",
                      "%d call(s) over %d blocks = %d rows of the workload with dZ and dW2, %.1f s wall, "
                      "fp64 C oracle, OpenMP over rows" % (calls, blocks, rows, el), threads)


def cpu_baseline_backward(inp, seconds: float, blocks: int = 16):
    import numpy as np
    import oracle
    import synth
    threads = cpu_threads()
    sub = synth.subset(inp, np.arange(blocks))
    rows = blocks * inp.gamma
    lo = oracle.block_loss(sub, want_dW2=False, nthreads=threads)
    calls, el = timed_repeats(lambda i: oracle.block_loss_backward(sub, lo["dZ"], lo["dA"], nthreads=threads),
                              seconds)
    return cpu_result(calls * rows / el, "rows/s",
                      "%d call(s) over %d blocks = %d rows of the workload (dW1, dw_conf, dh), %.1f s wall, "
                      "fp64 C oracle, OpenMP over rows" % (calls, blocks, rows, el), threads)


def cpu_baseline_verify(inp, tokens, logp, surv, target_bits, seconds: float):
    import oracle
    threads = cpu_threads()
    calls, el = timed_repeats(lambda i: oracle.verify_block(inp, tokens, logp, surv, target_bits, 0.25, seed=0,
                                                            offset=i, nthreads=threads), seconds)
    return cpu_result(calls * inp.B / el, "blocks/s",
                      "%d whole-batch call(s) of the workload (%d blocks), %.1f s wall, fp64 C oracle, "
                      "OpenMP over blocks" % (calls, inp.B, el), threads)


def copy_rate_gbs(dev) -> float:
    """A plain 1 GiB device-to-device copy timed with HIP events (read +
    write bytes over the time), best of 5: the attainable HBM rate."""
    import torch
    src = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = float("inf")
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        best = min(best, a.elapsed_time(b) * 1e-3)
    del src, dst
    return 2 * FLUSH_BYTES / best / 1e9


def copy_calibration() -> int:
    """A plain 1 GiB device-to-device copy, five times: reads and writes
    exactly 2^30 bytes per launch, the yardstick for the FETCH_SIZE and
    WRITE_SIZE counters."""
    import torch
    src = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": FLUSH_BYTES, "launches": 5}), flush=True)
    return 0


def run_timed(step, args, dev, kernels_per_call):
    """Warm-up, then args.steps calls each preceded by an untimed 1 GiB
    read, each bracketed by HIP events on the current stream (the value);
    then the same flushed calls again with the library's kernel timing
    switched on (its events would otherwise add to the calls' time); then
    the same number of calls back to back.  Returns per-call seconds
    (flushed), the warm wall time, and the library's per-launch kernel
    times (flushed calls, grouped per call)."""
    import torch
    from semi_autoregressive_draft_markov_amd import binding
    stream = torch.cuda.current_stream()
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    def flushed_calls(first):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            torch.sum(flush, dim=0, out=sink)  # reads 1 GiB: evicts the caches, leaves no dirty lines
            evs[i][0].record(stream)
            step(first + i)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e-3 for a, b in evs]

    call_s = flushed_calls(args.warmup)
    binding.dspark_profile_enable(True)
    binding.dspark_profile_read_each()
    flushed_calls(args.warmup + args.steps)
    each = binding.dspark_profile_read_each(capacity=args.steps * kernels_per_call + 16)
    binding.dspark_profile_enable(False)
    assert len(each) == args.steps * kernels_per_call, (len(each), args.steps, kernels_per_call)
    each_s = [ms * 1e-3 for ms in each]
    per_call = [each_s[i * kernels_per_call:(i + 1) * kernels_per_call] for i in range(args.steps)]
    del flush
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + 2 * args.steps + i)
    torch.cuda.synchronize()
    warm_s = time.perf_counter() - t0
    return call_s, warm_s, per_call


def base_line(metric, value, unit, args, ms_per_step, config, dtype="bf16"):
    return {"metric": metric, "value": round(value, 1), "unit": unit, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic", "config": config}


def timing_summary(call_s, warm_s, count_per_call, steps):
    return {"caches": "1 GiB read before every timed call",
            "call_us_median": round(statistics.median(call_s) * 1e6, 2),
            "call_us_min": round(min(call_s) * 1e6, 2),
            "warm_value": round(count_per_call * steps / warm_s, 1),
            "warm_ms_per_step": round(warm_s * 1e3 / steps, 4)}


def bench_draft(args) -> int:
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
    kname = binding.dspark_draft_kernel_name(dims)
    single = kname.startswith("k_draft_persistent")
    per_call = 1 if single else gamma

    def step(i):
        binding.dspark_draft_block(dims, t["U"], t["h"], t["anchor"], t["W1"], t["W2"], t["w_conf"],
                                   t["W_rnn"], t["temperature"], 0, i, out["tokens"], out["logp"],
                                   out["conf"], out["survival"], ws)

    call_s, warm_s, kernel_s = run_timed(step, args, dev, per_call)
    tokens = out["tokens"].cpu().numpy()
    assert np.all((tokens >= 0) & (tokens < V)), "bad tokens"
    elapsed = sum(call_s)
    avg_kernel_s = sum(sum(k) for k in kernel_s) / (args.steps * per_call)
    if single:
        # W2 once per call, every step's U slice once, the gathered W1 rows
        alg_bytes = (r + gamma * B) * V * 2 + gamma * B * r * 2
        alg_flops = 2.0 * gamma * B * r * V
        driver = "single-launch"
    else:
        # one launch per step: all of W2 plus the step's U slice
        alg_bytes = (r + B) * V * 2
        alg_flops = 2.0 * B * r * V
        driver = "per-step"
    names = {"qwen3-4b": "qwen3-4b-shaped markov-head block sampling",
             "qwen3-14b": "qwen3-14b-shaped markov-head block sampling, half greedy",
             "gemma4-rnn": "gemma4-12b-shaped rnn-head block sampling"}
    config = {"workload": names[args.workload], "V": V, "r": r, "d": d, "gamma": gamma, "B": B,
              "head": inp.head, "parallelism": "single-gpu"}
    line = base_line(METRIC, B * gamma * args.steps / elapsed, "tokens/s", args, elapsed * 1e3 / args.steps,
                     config)
    line["timing"] = timing_summary(call_s, warm_s, B * gamma, args.steps)
    line["roofline"] = roofline(args.workload, kname, avg_kernel_s, alg_bytes, alg_flops)
    line["roofline"]["driver"] = driver
    line["roofline"]["attainable_copy_GBps"] = round(copy_rate_gbs(dev), 1)
    line["cpu_baseline"] = cpu_baseline_draft(inp, args.cpu_seconds) if args.cpu_seconds > 0 else None
    print(json.dumps(line), flush=True)
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

    def step(i):
        binding.dspark_block_loss(dims, t["U"], t["target"], t["h"], t["anchor"], t["labels"],
                                  t["W1"], t["W2"], t["w_conf"], None, None, out["loss4"],
                                  out["c_star"], out["conf"], out["dlogits"], "bf16", out["dW2"],
                                  out["dconf_logit"], ws)

    # timed launches per call: passes 1, 2, 3 and the dW2 contraction
    call_s, warm_s, ks = run_timed(step, args, dev, 4)
    elapsed = sum(call_s)
    passes_s = sum(sum(k[:3]) for k in ks) / args.steps
    dw2_s = sum(k[3] for k in ks) / args.steps
    # the three passes' own inputs and outputs: passes 1 and 2 read U and T,
    # pass 3 reads U and writes bf16 dlogits (its sign bits from pass 2 are
    # an implementation detail and not counted); each recomputes the bias
    alg_bytes = 2 * (2 * R * V * 2) + 2 * R * V * 2
    gemm_flops = 2.0 * R * r * V
    config = {"workload": "qwen3-8b-shaped teacher-forced loss", "V": V, "r": r, "d": inp.d,
              "gamma": inp.gamma, "N": inp.B, "dlogits": "bf16"}
    line = base_line("teacher-forced rows/s (V=151936, r=256, γ=7, 7168 rows)", R * args.steps / elapsed,
                     "rows/s", args, elapsed * 1e3 / args.steps, config)
    line["timing"] = timing_summary(call_s, warm_s, R, args.steps)
    line["roofline"] = roofline("qwen3-8b-loss", "k_loss_mfma passes 1-3", passes_s, alg_bytes, 3 * gemm_flops,
                                match=["k_loss_mfma<"])
    # dW2 = E^T dZ: bf16 dZ and W2-shaped output, against the matrix cores
    dw2_bytes = R * V * 2 + r * V * 4 + r * R * 2
    line["dw2"] = roofline("qwen3-8b-loss", "k_dw2_mfma<0>", dw2_s, dw2_bytes, gemm_flops)
    line["dw2"]["mfma_tflops"] = round(gemm_flops / dw2_s / 1e12, 1)
    line["roofline"]["attainable_copy_GBps"] = round(copy_rate_gbs(dev), 1)
    line["cpu_baseline"] = cpu_baseline_loss(inp, args.cpu_seconds) if args.cpu_seconds > 0 else None
    print(json.dumps(line), flush=True)
    return 0


def bench_backward(args) -> int:
    """Backward past the logits over the Qwen3-8B-shaped workload (7168 rows,
    V = 151936, r = 256, d = 4096): one dspark_block_loss call makes bf16
    dlogits and dconf_logit, then a step is one dspark_block_loss_backward
    call (dW1, dw_conf, dh)."""
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

    def step(i):
        binding.dspark_block_loss_backward(dims, lo["dlogits"], "bf16", lo["dconf_logit"], t["h"],
                                           t["anchor"], t["labels"], t["W1"], t["W2"],
                                           t["w_conf"], out["dW1"], out["dw_conf"], out["dh"], ws)

    call_s, warm_s, ks = run_timed(step, args, dev, 1)
    elapsed = sum(call_s)
    de_s = sum(k[0] for k in ks) / args.steps
    alg_bytes = R * V * 2 + r * V * 2
    flops = 2.0 * R * V * r
    config = {"workload": "qwen3-8b-shaped backward past the logits", "V": V, "r": r, "d": d,
              "gamma": inp.gamma, "N": inp.B, "dlogits": "bf16"}
    line = base_line("teacher-forced rows/s through the backward past the logits (V=151936, r=256, d=4096, "
                     "7168 rows)", R * args.steps / elapsed, "rows/s", args, elapsed * 1e3 / args.steps, config)
    line["timing"] = timing_summary(call_s, warm_s, R, args.steps)
    line["roofline"] = roofline("qwen3-8b-backward", "k_de_mfma<8, 2, false>", de_s, alg_bytes, flops)
    line["roofline"]["attainable_copy_GBps"] = round(copy_rate_gbs(dev), 1)
    line["cpu_baseline"] = cpu_baseline_backward(inp, args.cpu_seconds) if args.cpu_seconds > 0 else None
    print(json.dumps(line), flush=True)
    return 0


def bench_verify(args) -> int:
    """Verification of Qwen3-4B-shaped drafted blocks (B = 32, gamma = 7,
    V = 151936, r = 256, bf16): one dspark_draft_block call drafts the
    blocks, synthetic target logits [B, gamma + 1, V] (the base logits plus
    N(0, 0.3^2) at the drafted positions) stand in for the target model;
    a step is one dspark_verify_block call (threshold 0.25)."""
    import numpy as np
    import torch

    import synth
    from semi_autoregressive_draft_markov_amd import binding, ops

    binding.load()
    dev = torch.device("cuda:0")
    inp = synth.config_inputs(2)
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

    call_s, warm_s, ks = run_timed(step, args, dev, 1)
    elapsed = sum(call_s)
    k_s = sum(k[0] for k in ks) / args.steps
    alg_bytes = r * V * 2 + B * V * 2 + B * V * 4
    flops = 2.0 * B * r * V
    acc = out["n_accept"].float().mean().item()
    config = {"workload": "qwen3-4b-shaped verification of drafted blocks", "V": V, "r": r, "gamma": gamma,
              "B": B, "threshold": 0.25, "mean_accepted": round(acc, 3)}
    line = base_line("verified blocks/s (V=151936, r=256, γ=7, B=32)", B * args.steps / elapsed, "blocks/s",
                     args, elapsed * 1e3 / args.steps, config)
    line["timing"] = timing_summary(call_s, warm_s, B, args.steps)
    line["roofline"] = roofline("qwen3-4b-verify", "k_v_bias_mfma<8>", k_s, alg_bytes, flops)
    line["roofline"]["attainable_copy_GBps"] = round(copy_rate_gbs(dev), 1)
    if args.cpu_seconds > 0:
        tgt_bits = tgt.view(torch.int16).cpu().numpy().view(np.uint16)
        line["cpu_baseline"] = cpu_baseline_verify(inp, d["tokens"].cpu().numpy(),
                                                   d["logp"].cpu().numpy().astype(np.float64),
                                                   d["survival"].cpu().numpy().astype(np.float64), tgt_bits,
                                                   args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


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
    ap.add_argument("--copy-calibration", action="store_true",
                    help="instead of the benchmark, run a plain device copy of 1 GiB "
                         "(reference for HBM byte counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        return copy_calibration()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library runs the drafting path on a single GPU "
              "(blocks are independent; sharding them over GPUs is not implemented); run it with --gpus 1",
              file=sys.stderr)
        return 2
    if args.workload == "qwen3-8b-loss":
        return bench_loss(args)
    if args.workload == "qwen3-8b-backward":
        return bench_backward(args)
    if args.workload == "qwen3-4b-verify":
        return bench_verify(args)
    return bench_draft(args)


if __name__ == "__main__":
    sys.exit(main())
