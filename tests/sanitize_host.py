"""Host-sanitizer run of the library's CPU code (slot manager, decode-step driver, host expert).

Builds every source of libmoe with AddressSanitizer and UndefinedBehaviorSanitizer on the host
pass only (device code is compiled as usual), links it to _build/asan/libmoe.so, and runs the
CPU tests that drive the host code through the C ABI -- the slot cache and its policy mode, the
host expert with its thread pool, argument validation of every entry point -- against that build
(MOE_LIB_PATH), with the sanitizer runtime preloaded into Python.  Any report ends the run with a
non-zero status.

    python tests/sanitize_host.py            # build, then run the tests
    python tests/sanitize_host.py --no-build # run against an existing sanitizer build

No GPU is needed or used.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from expert_offload_cache_amd import build as b  # noqa: E402

OUT_DIR = os.path.join(ROOT, "_build", "asan")
LIB = os.path.join(OUT_DIR, "libmoe.so")
TESTS = ["tests/test_cache_host.py", "tests/test_cpu_expert.py", "tests/test_abi.py"]
# host-pass only: every sanitizer flag goes through -Xarch_host
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]


def runtime() -> str:
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang's AddressSanitizer runtime was not found under /opt/rocm/llvm")
    return hits[-1]


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    cmd = [b.HIPCC, *b.FLAGS, *HOST_SAN, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-4000:]}")
    return obj


def build() -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = b.sources()
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(_compile, srcs))
    subprocess.run([b.HIPCC, f"--offload-arch={b.ARCH}", "-shared", "-fPIC", *HOST_SAN,
                    "-Xarch_host", "-shared-libsan", *objs, "-o", LIB], check=True)
    return LIB


def run_tests() -> int:
    env = dict(os.environ)
    env.update(MOE_LIB_PATH=LIB, LD_PRELOAD=runtime(),
               # Python's own allocations are not freed at exit: leak checking stays off
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=87")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider", *TESTS]
    return subprocess.run(cmd, cwd=ROOT, env=env).returncode


if __name__ == "__main__":
    if "--no-build" not in sys.argv:
        print("building", build(), flush=True)
    rc = run_tests()
    print("sanitizer run:", "clean" if rc == 0 else f"FAILED (status {rc})", flush=True)
    sys.exit(rc)
