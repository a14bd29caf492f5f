"""Build libgqa.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libgqa.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found")
    return exe


def kernels_using_scratch(remarks):
    """Kernels whose resource-usage remark reports scratch (private) memory per lane."""
    found, name = [], None
    for line in remarks.splitlines():
        line = line.split(" [-Rpass", 1)[0]  # drop the trailing flag name
        if "Function Name:" in line:
            name = line.split("Function Name:", 1)[1].strip()
        elif "ScratchSize [bytes/lane]:" in line and name is not None:
            size = int(line.rsplit(":", 1)[1])
            if size > 0:
                found.append((name, size))
    return found


def build_library(verbose=False, extra_flags=()):
    srcs = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))
    tmp = LIB + ".tmp"
    # the resource-usage remarks let the build refuse kernels that spill to scratch memory: on gfx950 a
    # kernel with scratch also slowed the decode kernel launched after it
    cmd = ([hipcc()] + HIPCC_FLAGS + list(extra_flags) + ["-Rpass-analysis=kernel-resource-usage",
           "-I", os.path.join(ROOT, "include"), "-o", tmp] + srcs)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libgqa.so")
    scratch = kernels_using_scratch(res.stderr)
    if scratch:
        os.remove(tmp)
        raise RuntimeError("kernels use scratch memory: " + ", ".join(f"{n} ({b} B/lane)" for n, b in scratch))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
