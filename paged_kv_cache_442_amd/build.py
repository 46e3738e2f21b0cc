"""Build ``libpa.so`` in-tree with hipcc for gfx950.

``python -m paged_kv_cache_442_amd.build`` (or ``build_library()``) always recompiles.
The library is written next to this file; the ctypes binding loads it from there.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libpa.so")

SOURCES = ["capi.cpp", "block_manager.cpp", "kernels.hip", "prefill.hip"]

# Packed-FP32 VALU forms are kept out of the generated code on purpose; the host
# pass warns that it does not know the feature, which is harmless.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    # A single-lane atomic stays a single-lane atomic (the wave-aggregating rewrite
    # needs the result at once, which would stall the decode kernel's load pipeline).
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build libpa.so)")
    return path


def build_library(verbose=False):
    """Compile every source into ``libpa.so`` (atomically replaced); returns its path."""
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIP_FLAGS + ["-I", INCLUDE, "-I", CSRC] + \
        [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed (%d):\n%s\n%s" % (res.returncode, res.stdout, res.stderr))
    noise = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if verbose and noise:
        print("\n".join(noise), file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
