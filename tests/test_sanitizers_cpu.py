"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The library's host side -- argument validation and workspace arithmetic of
the C ABI, STS and the prefix scheduler -- and the C oracle are rebuilt with
clang's ASan + UBSan (device code unchanged: the sanitizer flags apply to
the host compilation only), then the CPU tests that exercise them run in a
child process with the ASan runtime preloaded.  Any sanitizer report fails
the test.  No GPU is used."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"


def asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


# host-only sanitizer flags for hipcc: each -fsanitize= right after -Xarch_host
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-shared-libasan"]


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    rt = asan_runtime()
    if rt is None or not os.path.exists(CLANG):
        pytest.skip("clang's ASan runtime is not installed")
    d = tmp_path_factory.mktemp("sanitized")
    sys.path.insert(0, ROOT)
    from semi_autoregressive_draft_markov_amd import build
    lib = build.build(extra_flags=HOST_SANITIZE, out=str(d / "libdspark_asan.so"))
    orc = str(d / "liboracle_asan.so")
    subprocess.run([CLANG, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-shared-libasan",
                    os.path.join(ROOT, "oracle", "dspark_oracle.c"), "-o", orc, "-lm"], check=True)
    return rt, lib, orc


def run_sanitized(sanitized, tests):
    rt, lib, orc = sanitized
    env = dict(os.environ, LD_PRELOAD=rt, DSPARK_LIBRARY=lib, DSPARK_ORACLE_LIBRARY=orc,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider"]
                         + [os.path.join(ROOT, "tests", t) for t in tests],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    return out


def test_sanitized_builds_are_instrumented_and_loaded(sanitized):
    rt, lib, orc = sanitized
    for so in (lib, orc):
        syms = subprocess.run(["nm", "-D", so], capture_output=True, text=True, check=True).stdout
        assert "__asan_report_load" in syms and "__ubsan_handle" in syms, so
    probe = ("import ctypes, oracle\n"
             "from semi_autoregressive_draft_markov_amd import binding\n"
             "binding.load(); oracle._load()\n"
             "maps = open('/proc/self/maps').read()\n"
             "assert binding.LIB_PATH in maps and oracle._LIB in maps\n"
             "ctypes.CDLL(None).__asan_init\n"
             "print('instrumented')\n")
    env = dict(os.environ, LD_PRELOAD=rt, DSPARK_LIBRARY=lib, DSPARK_ORACLE_LIBRARY=orc,
               ASAN_OPTIONS="detect_leaks=0")
    res = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=300)
    assert res.returncode == 0 and "instrumented" in res.stdout, res.stdout + res.stderr


def test_library_host_code_under_sanitizers(sanitized):
    out = run_sanitized(sanitized, ["test_abi_cpu.py", "test_host_sched.py"])
    assert " passed" in out


def test_oracle_under_sanitizers(sanitized):
    out = run_sanitized(sanitized, ["test_oracle_philox.py", "test_oracle_loss.py", "test_oracle_verify.py",
                                    "test_oracle_sampling.py"])
    assert " passed" in out
