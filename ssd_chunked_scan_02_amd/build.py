"""Build libssd.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIBRARY = os.path.join(PKG, "libssd.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Device code: no packed-fp32 instructions (the compiler would otherwise form them from
# scalar float code).
DEVICE_FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Wall", "-Wno-unused-result"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall"]
DEVICE_SOURCES = ["ssd_kernels.hip", "ssd_fast.hip", "ssd_diag.hip", "ssd_bwd.hip", "ssd_noalloc.hip"]


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature flag; that warning is noise.
    out = "\n".join(l for l in proc.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "unknown target feature" not in l)
    if proc.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("command failed: " + " ".join(cmd))
    return out


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel) and link libssd.so next to this file; returns its path."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(BUILD_DIR, exist_ok=True)
    inc = ["-I", INCLUDE, "-I", CSRC]
    cmds, objs = [], []
    for src in DEVICE_SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        cmds.append([HIPCC, *DEVICE_FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    a_obj = os.path.join(BUILD_DIR, "ssd_api.o")
    cmds.append([HIPCC, *HOST_FLAGS, *inc, "-c", os.path.join(CSRC, "ssd_api.cpp"), "-o", a_obj])
    jobs = max(1, min(len(cmds), len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        logs = list(pool.map(_run, cmds))
    tmp = LIBRARY + ".tmp%d" % os.getpid()
    logs.append(_run([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, a_obj, "-o", tmp]))
    os.replace(tmp, LIBRARY)
    if verbose:
        for log in logs:
            if log.strip():
                print(log)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
