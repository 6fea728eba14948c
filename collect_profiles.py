#!/usr/bin/env python3
"""Collect the rocprofv3 evidence behind bench.py's roofline lines.

For every workload bench.py knows this runs, one child process each:

  * one kernel trace with statistics (`--kernel-trace --stats`) of a short
    bench run, for the per-kernel average durations;
  * four counter passes of a shorter bench run: FETCH_SIZE, WRITE_SIZE and
    two sets of SQ/GRBM counters (each pass within the per-block limits of
    one rocprofv3 run);

and two counter passes (FETCH_SIZE, WRITE_SIZE) of a plain 1 GiB device
copy (`bench.py --copy-calibration`), which scale the byte counters to
bytes.  Every pass runs under its own `timeout -s KILL`.

Output (default prof_out/profiles/): counters.json -- per workload and
kernel the per-dispatch averages of every counter, tagged with the hash of
the kernel sources they were taken on -- and one markdown summary per
workload with the commands, the kernel table and the derived figures.
Raw rocprofv3 output stays under prof_out/raw/ (neither is kept in the
repository; the summaries are copied into profiles/).

`--merge A.json B.json ... --out DIR` (no GPU) joins counters.json files of
separate runs over different workloads, taken on the same kernel sources,
into DIR/counters.json (for runs that do not fit one time limit together).
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (constants and the source hash only; no GPU work at import)

WORKLOADS = ["qwen3-4b", "qwen3-14b", "gemma4-rnn", "qwen3-8b-loss", "qwen3-8b-backward", "qwen3-4b-verify"]
TITLES = {
    "qwen3-4b": "Qwen3-4B-shaped Markov-head sampling (V 151936, r 256, d 2560, B 32, γ 7, bf16, T = 1)",
    "qwen3-14b": "Qwen3-14B-shaped Markov-head drafting, half the blocks greedy (V 151936, r 256, B 256, γ 7)",
    "gemma4-rnn": "Gemma4-12B-shaped RNN-head sampling (V 262144, r 256, B 128, γ 7)",
    "qwen3-8b-loss": "Qwen3-8B-shaped teacher-forced loss (7168 rows, V 151936, r 256, d 4096, bf16 dlogits)",
    "qwen3-8b-backward": "Qwen3-8B-shaped backward past the logits (7168 rows, V 151936, r 256, d 4096)",
    "qwen3-4b-verify": "Qwen3-4B-shaped verification of drafted blocks (B 32, γ 7, V 151936, r 256)",
}
PASSES = [
    ("fetch", ["FETCH_SIZE"]),
    ("write", ["WRITE_SIZE"]),
    ("sq1", ["SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES",
             "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU"]),
    ("sq2", ["SQ_ACTIVE_INST_ANY", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_WAIT_ANY",
             "SQ_INSTS_VMEM", "SQ_ACTIVE_INST_LDS", "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE"]),
]
XCDS = 8    # GRBM_GUI_ACTIVE is summed over the XCDs
SIMDS = 256 * 4


def short_name(full: str) -> str:
    """'void dspark::k_x<8, true>(dspark::Args)' -> 'k_x<8, true>'."""
    s = full.strip()
    if s.startswith("void "):
        s = s[5:]
    depth = 0
    for i, ch in enumerate(s):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            s = s[:i]
            break
    return s.replace("dspark::", "").strip()


def find_one(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise RuntimeError("no *%s under %s" % (suffix, d))
    return hits[-1]


def col(row: dict, *names):
    for n in names:
        for k in row:
            if k.lower() == n.lower():
                return row[k]
    raise KeyError(names)


def per_dispatch(csv_path: str) -> dict:
    """{kernel: {counter: mean per dispatch, '_dispatches': n}} from a
    rocprofv3 counter-collection CSV (one row per dispatch and counter)."""
    sums, disp = {}, {}
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            k = short_name(col(row, "Kernel_Name"))
            c = col(row, "Counter_Name")
            v = float(col(row, "Counter_Value"))
            d = col(row, "Dispatch_Id", "Dispatch_ID")
            sums.setdefault(k, {}).setdefault(c, 0.0)
            sums[k][c] += v
            disp.setdefault(k, set()).add(d)
    out = {}
    for k, cs in sums.items():
        n = len(disp[k])
        out[k] = {c: v / n for c, v in cs.items()}
        out[k]["_dispatches"] = n
    return out


def kernel_stats(csv_path: str) -> list:
    rows = []
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            rows.append({"kernel": short_name(col(row, "Name", "KernelName", "Kernel_Name")),
                         "calls": int(float(col(row, "Calls"))),
                         "total_us": float(col(row, "TotalDurationNs")) / 1e3,
                         "avg_us": float(col(row, "AverageNs")) / 1e3,
                         "pct": float(col(row, "Percentage"))})
    return rows


def run(cmd: list, log: str, limit: int) -> str:
    print("pass: %s" % " ".join(cmd), flush=True)
    os.makedirs(os.path.dirname(log), exist_ok=True)
    t0 = time.time()
    env = dict(os.environ, TMPDIR="/tmp")
    with open(log, "w") as f:
        res = subprocess.run(["timeout", "-s", "KILL", str(limit)] + cmd, cwd="/tmp", env=env, stdout=subprocess.PIPE,
                             stderr=f, text=True)
    with open(log, "a") as f:
        f.write(res.stdout)
    print("  rc %d, %.1f s" % (res.returncode, time.time() - t0), flush=True)
    if res.returncode != 0:
        raise RuntimeError("%s failed with %d (log %s)" % (cmd[0], res.returncode, log))
    return res.stdout


def bench_cmd(workload: str, steps: int, warmup: int) -> list:
    return ["python3", os.path.join(ROOT, "bench.py"), "--workload", workload, "--steps", str(steps), "--warmup",
            str(warmup), "--cpu-seconds", "0"]


def rel(p: str) -> str:
    return os.path.relpath(p, ROOT)


def show(cmd: list) -> str:
    return " ".join(rel(c) if c.startswith(ROOT) else c for c in cmd)


def derived(c: dict) -> dict:
    """Per-launch figures from one kernel's counters (cycles per XCD from
    GRBM_GUI_ACTIVE; SQ cycle counters are in units of 4 cycles except the
    MFMA busy count)."""
    out = {}
    cyc = c.get("GRBM_GUI_ACTIVE", 0.0) / XCDS
    if cyc > 0:
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
            out["mfma_util_pct"] = round(100.0 * c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * SIMDS), 2)
        if "SQ_ACTIVE_INST_VALU" in c:
            out["valu_busy_pct"] = round(100.0 * 4 * c["SQ_ACTIVE_INST_VALU"] / (cyc * SIMDS), 2)
    if c.get("SQ_ACTIVE_INST_LDS"):
        out["lds_bank_conflict_per_lds_cycle"] = round(c.get("SQ_LDS_BANK_CONFLICT", 0.0) / c["SQ_ACTIVE_INST_LDS"], 3)
    if c.get("SQ_WAVE_CYCLES"):
        out["wait_any_per_wave_cycle"] = round(c.get("SQ_WAIT_ANY", 0.0) / c["SQ_WAVE_CYCLES"], 3)
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--workloads", default=",".join(WORKLOADS))
    ap.add_argument("--out", default=os.path.join(ROOT, "prof_out", "profiles"))
    ap.add_argument("--raw", default=os.path.join(ROOT, "prof_out", "raw"))
    ap.add_argument("--trace-steps", type=int, default=20)
    ap.add_argument("--pmc-steps", type=int, default=3)
    ap.add_argument("--merge", nargs="+", help="counters.json files to join (no GPU work)")
    args = ap.parse_args()
    # (the passes run with /tmp as working directory)
    args.out, args.raw = os.path.abspath(args.out), os.path.abspath(args.raw)
    if args.merge:
        return merge(args.merge, args.out)
    os.makedirs(args.out, exist_ok=True)
    os.makedirs(args.raw, exist_ok=True)
    result = {"kernel_source_hash": bench.kernel_source_hash(), "workloads": {}, "commands": {}}

    # the yardstick: a plain 1 GiB copy reads and writes 2^30 bytes per launch
    cal = {}
    for name, ctr in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        d = os.path.join(args.raw, "copy_" + name)
        cmd = ["rocprofv3", "--pmc", ctr, "--output-format", "csv", "-d", d, "-o", name, "--",
               "python3", os.path.join(ROOT, "bench.py"), "--copy-calibration"]
        run(cmd, d + ".log", 120)
        pd = per_dispatch(find_one(d, "counter_collection.csv"))
        copies = [v for k, v in pd.items() if "copy" in k.lower() or "elementwise" in k.lower()]
        if not copies:
            raise RuntimeError("no copy kernel in %s" % sorted(pd))
        best = max(copies, key=lambda v: v.get(ctr, 0.0))
        cal[name] = best[ctr] * (1 << 30) / bench.FLUSH_BYTES
        result["commands"].setdefault("copy_calibration", []).append(show(cmd))
    result["copy_calibration"] = {"fetch_kib_per_gib": cal["fetch"], "write_kib_per_gib": cal["write"]}

    for w in [x for x in args.workloads.split(",") if x]:
        cmds = []
        d = os.path.join(args.raw, w, "trace")
        tcmd = ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d", d, "-o", "trace", "--"] + \
            bench_cmd(w, args.trace_steps, 3)
        out = run(tcmd, d + ".log", 600)
        cmds.append(show(tcmd))
        line = json.loads([l for l in out.splitlines() if l.startswith("{")][-1])
        stats = kernel_stats(find_one(d, "kernel_stats.csv"))
        counters = {}
        for name, ctrs in PASSES:
            d = os.path.join(args.raw, w, name)
            cmd = ["rocprofv3", "--pmc"] + ctrs + ["--output-format", "csv", "-d", d, "-o", name, "--"] + \
                bench_cmd(w, args.pmc_steps, 1)
            run(cmd, d + ".log", 300)
            cmds.append(show(cmd))
            for k, v in per_dispatch(find_one(d, "counter_collection.csv")).items():
                n = v.pop("_dispatches")
                counters.setdefault(k, {}).update(v)
                counters[k]["_dispatches_" + name] = n
        kern = {}
        for k, v in counters.items():
            if k.startswith("k_") or k.startswith("dspark"):
                e = {"fetch_kib": v.get("FETCH_SIZE"), "write_kib": v.get("WRITE_SIZE"),
                     "sq_insts_valu": v.get("SQ_INSTS_VALU")}
                e.update(derived(v))
                e["raw"] = {c: round(x, 1) for c, x in sorted(v.items())}
                kern[k] = e
        result["workloads"][w] = {"kernels": kern, "kernel_stats": stats, "bench_line": line}
        result["commands"][w] = cmds
        write_summary(args.out, w, line, stats, kern, cmds, result)
    with open(os.path.join(args.out, "counters.json"), "w") as f:
        json.dump(result, f, indent=1, sort_keys=True)
    print("wrote %s" % os.path.join(args.out, "counters.json"), flush=True)
    return 0


def merge(files, out_dir) -> int:
    parts = [json.load(open(f)) for f in files]
    hashes = {p["kernel_source_hash"] for p in parts}
    if len(hashes) != 1:
        raise SystemExit("counter files taken on different kernel sources: %s" % sorted(hashes))
    result = {"kernel_source_hash": hashes.pop(), "workloads": {}, "commands": {},
              "copy_calibration": parts[0]["copy_calibration"]}
    for p in parts:
        for w, v in p["workloads"].items():
            if w in result["workloads"]:
                raise SystemExit("workload %s appears in more than one file" % w)
            result["workloads"][w] = v
        for k, v in p["commands"].items():
            if k != "copy_calibration" or k not in result["commands"]:
                result["commands"][k] = v
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, "counters.json"), "w") as f:
        json.dump(result, f, indent=1, sort_keys=True)
    print("wrote %s (%s)" % (os.path.join(out_dir, "counters.json"), ", ".join(sorted(result["workloads"]))))
    return 0


def write_summary(out_dir, w, line, stats, kern, cmds, result):
    roof = line.get("roofline", {})
    main_kernel = roof.get("kernel", "")
    base = main_kernel.split("<")[0].split(" ")[0] or "kernels"
    fs = (1 << 30) / 1024.0 / result["copy_calibration"]["fetch_kib_per_gib"]
    ws = (1 << 30) / 1024.0 / result["copy_calibration"]["write_kib_per_gib"]
    L = ["# %s — %s" % (main_kernel or base, TITLES.get(w, w)), ""]
    L.append("Made by `python3 collect_profiles.py --workloads %s` (kernel sources %s), which ran:" %
             (w, result["kernel_source_hash"]))
    L.append("")
    L.append("    cd /tmp && export TMPDIR=/tmp")
    for c in cmds:
        L.append("    " + c)
    for c in result["commands"].get("copy_calibration", []):
        L.append("    " + c)
    L += ["", "Kernel trace (`--kernel-trace --stats`):", "", "| kernel | calls | total µs | avg µs | % |",
          "|---|---|---|---|---|"]
    for s in stats:
        L.append("| %s | %d | %.1f | %.2f | %.1f |" % (s["kernel"], s["calls"], s["total_us"], s["avg_us"], s["pct"]))
    L += ["", "bench.py line of the traced run (live HIP-event timing; the trace itself slows calls slightly):", "",
          "    " + json.dumps({k: line.get(k) for k in ("value", "unit", "ms_per_step")}),
          "    roofline: " + json.dumps({k: roof.get(k) for k in ("bound", "achieved", "unit", "frac", "kernel",
                                                                     "kernel_us", "fractions")}), ""]
    L += ["Counters per dispatch (averaged over the dispatches of the counter runs); HBM bytes = FETCH_SIZE × "
          "%.4f + WRITE_SIZE × %.4f KiB, the factors that map a 1 GiB device copy's counts to 2^30 bytes:" % (fs, ws),
          "", "| kernel | FETCH KiB | WRITE KiB | HBM MB | VALU insts | VALU busy % | MFMA util % | LDS conflict / "
          "LDS cycle | wait / wave cycle |", "|---|---|---|---|---|---|---|---|---|"]
    for k, e in sorted(kern.items()):
        mb = ((e["fetch_kib"] or 0) * fs + (e["write_kib"] or 0) * ws) * 1024 / 1e6
        L.append("| %s | %.1f | %.1f | %.2f | %.0f | %s | %s | %s | %s |" % (
            k, e["fetch_kib"] or 0, e["write_kib"] or 0, mb, e["sq_insts_valu"] or 0, e.get("valu_busy_pct", "-"),
            e.get("mfma_util_pct", "-"), e.get("lds_bank_conflict_per_lds_cycle", "-"),
            e.get("wait_any_per_wave_cycle", "-")))
    L.append("")
    with open(os.path.join(out_dir, "%s_%s.md" % (base, w)), "w") as f:
        f.write("\n".join(L))


if __name__ == "__main__":
    sys.exit(main())
