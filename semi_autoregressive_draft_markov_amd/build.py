"""Build the gfx950 HIP library libdspark.so in-tree with hipcc.

Every source in csrc/ is compiled to its own object in parallel (one hipcc
per file), then the objects are linked into libdspark.so.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdspark.so")
OBJ_DIR = os.path.join(HERE, "_build")
ARCH = os.environ.get("DSPARK_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    "--offload-arch=" + ARCH,
    # packed-fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-parameter", "-Wno-unused-function",
]
NOISE = "is not a recognized feature for this target"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if NOISE not in l)
    return res.returncode, err


def _jobs() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 4)
    return max(1, min(n, 16))


def build(verbose: bool = False, extra_flags=(), out: str = LIB) -> str:
    """Compile every csrc/*.hip (and the host-only csrc/*.cpp) into `out`
    (libdspark.so by default); always recompiles."""
    obj_dir = OBJ_DIR if out == LIB else os.path.join(os.path.dirname(os.path.abspath(out)), "_build")
    if os.path.isdir(obj_dir):
        shutil.rmtree(obj_dir)
    os.makedirs(obj_dir)
    srcs = sources()
    objs = [os.path.join(obj_dir, os.path.basename(s) + ".o") for s in srcs]
    flags = HIPCC_FLAGS + list(extra_flags)
    cmds = [[hipcc()] + flags + ["-c", s, "-o", o] for s, o in zip(srcs, objs)]
    with ThreadPoolExecutor(max_workers=_jobs()) as pool:
        results = list(pool.map(_run, cmds))
    errs = [(s, e) for s, (rc, e) in zip(srcs, results) if rc != 0]
    if errs:
        raise RuntimeError("hipcc failed:\n" + "\n".join("%s:\n%s" % (s, e) for s, e in errs))
    if verbose:
        for s, (_, e) in zip(srcs, results):
            if e.strip():
                print(e, file=sys.stderr)
    tmp = out + ".tmp%d" % os.getpid()
    rc, err = _run([hipcc()] + flags + ["-shared"] + objs + ["-o", tmp])
    if rc != 0:
        raise RuntimeError("hipcc link failed:\n" + err)
    os.replace(tmp, out)
    shutil.rmtree(obj_dir, ignore_errors=True)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
