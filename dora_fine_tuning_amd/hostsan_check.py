"""CPU check of the C ABI's host code under AddressSanitizer and
UndefinedBehaviorSanitizer.

Builds libdora_hip_hostsan.so (host code instrumented, device code as in the
product) and runs tests/test_abi_cpu.py against it in a child process with the
ASan runtime preloaded (ahead of anything already in LD_PRELOAD).  Leak
detection is off: the Python interpreter itself holds memory until exit.  Any
sanitizer report aborts the child, so a clean run is exit status 0.

    python -m dora_fine_tuning_amd.hostsan_check
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def asan_runtime() -> str:
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise FileNotFoundError("clang's shared ASan runtime (libclang_rt.asan-x86_64.so) not found under /opt/rocm")
    return hits[-1]


def main() -> int:
    from dora_fine_tuning_amd import build

    lib = build.build(sanitize=True)
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = asan_runtime() + (":" + pre if pre else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["DORA_HIP_LIB"] = lib
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_abi_cpu.py")]
    print("running:", " ".join(cmd), f"(DORA_HIP_LIB={lib})", flush=True)
    return subprocess.call(cmd, cwd=ROOT, env=env)


if __name__ == "__main__":
    sys.exit(main())
