"""Build the HIP library libdora_hip.so in-tree with hipcc for gfx950.

Every source under csrc/ is compiled to an object in parallel and linked into
one shared library next to this file.  Packed fp32 instructions are disabled
(-packed-fp32-ops) for all device code.  The build fails if any kernel spills
registers to scratch memory (read from the compiler's resource-usage remarks):
a spill in a streaming kernel costs far more than the registers it saves.
"""
from __future__ import annotations

import glob
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdora_hip.so")
ROOT = os.path.dirname(HERE)

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


RESOURCE_REMARKS = ["-Rpass-analysis=kernel-resource-usage"]
_FUNC = re.compile(r"remark: Function Name: (\S+)")
_SCRATCH = re.compile(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)")


def _spills(log: str) -> tuple[list[str], str]:
    """(kernels with scratch > 0, the log without the resource remarks)."""
    bad, kept, func = [], [], None
    for line in log.splitlines():
        m = _FUNC.search(line)
        if m:
            func = m.group(1)
        m = _SCRATCH.search(line)
        if m and int(m.group(1)) > 0:
            bad.append(f"{func}: {m.group(1)} bytes/lane")
        if "kernel-resource-usage" not in line:
            kept.append(line)
    return bad, "\n".join(kept)


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for a CPU check of
# the C ABI's validation layer: every -fsanitize= goes to the host compilation
# only (-Xarch_host); the device code is built exactly as in the product.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
SANITIZED_LIB = os.path.join(HERE, "libdora_hip_hostsan.so")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every csrc/*.hip and link libdora_hip.so; returns its path.
    With ``sanitize`` the host code is instrumented (see SANITIZE) and the
    result goes to libdora_hip_hostsan.so, for CPU tests only."""
    srcs = sources()
    flags = COMMON + (SANITIZE if sanitize else [])
    lib = SANITIZED_LIB if sanitize else LIB
    tmp = tempfile.mkdtemp(prefix="dora_build_")
    try:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in srcs]
        with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
            logs = list(ex.map(lambda so: _run([HIPCC, *flags, *RESOURCE_REMARKS, "-c", so[0], "-o", so[1]]),
                               zip(srcs, objs)))
        spilled = []
        for i, l in enumerate(logs):
            bad, logs[i] = _spills(l)
            spilled += bad
        if spilled:
            raise RuntimeError("kernels spill to scratch memory:\n  " + "\n  ".join(spilled))
        tmp_lib = lib + ".tmp"
        logs.append(_run([HIPCC, *flags, "-shared", "-o", tmp_lib, *objs]))
        os.replace(tmp_lib, lib)
        if verbose:
            for l in logs:
                if l.strip():
                    print(l)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
