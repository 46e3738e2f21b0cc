"""Build ``libpa.so``, its debug twin ``libpa_debug.so`` and the read-bandwidth probes
``libpa_probe.so`` (bench.py's measured ceilings) in-tree with hipcc for gfx950.

``python -m paged_kv_cache_442_amd.build`` (or ``build_library()``) always recompiles.
Each source is compiled once to an object (in parallel); the C-ABI layer is compiled
twice, the second time with ``-DPA_DEBUG`` (host-side precondition checks of the
caller's slots and copy pairs before each launch), and the two libraries are linked
from those objects.  Both are written next to this file; the ctypes binding loads
``libpa.so`` from there.
"""

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libpa.so")
DEBUG_LIB_PATH = os.path.join(HERE, "libpa_debug.so")
# Read-bandwidth probes for bench.py's measured ceilings (not part of the attention path).
PROBE_LIB_PATH = os.path.join(HERE, "libpa_probe.so")

SOURCES = ["capi.cpp", "block_manager.cpp", "preconditions.cpp", "kernels.hip", "prefill.hip"]

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


def _run_all(cmds, verbose):
    procs = []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    errors = []
    for cmd, p in zip(cmds, procs):
        out, err = p.communicate()
        if p.returncode != 0:
            errors.append("%s failed (%d):\n%s\n%s" % (" ".join(cmd[-3:]), p.returncode, out, err))
        noise = [ln for ln in err.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if verbose and noise:
            print("\n".join(noise), file=sys.stderr)
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errors))


def build_library(verbose=False):
    """Compile every source and link ``libpa.so`` and ``libpa_debug.so`` (each atomically
    replaced); returns the path of ``libpa.so``."""
    compile_flags = [f for f in HIP_FLAGS if f != "-shared"]
    with tempfile.TemporaryDirectory(prefix="pa_build_") as tmp:
        objs, cmds = {}, []
        for src in SOURCES + ["capi.cpp#debug", "probes.hip"]:
            name, _, variant = src.partition("#")
            obj = os.path.join(tmp, name.replace(".", "_") + ("_debug" if variant else "") + ".o")
            extra = ["-DPA_DEBUG"] if variant else []
            cmds.append([hipcc()] + compile_flags + extra + ["-I", INCLUDE, "-I", CSRC, "-c",
                                                            os.path.join(CSRC, name), "-o", obj])
            objs[src] = obj
        _run_all(cmds, verbose)
        links = []
        for path, capi in ((LIB_PATH, "capi.cpp"), (DEBUG_LIB_PATH, "capi.cpp#debug")):
            members = [objs[capi]] + [objs[s] for s in SOURCES if s != "capi.cpp"]
            links.append([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + members +
                         ["-o", path + ".tmp%d" % os.getpid()])
        links.append([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", objs["probes.hip"],
                      "-o", PROBE_LIB_PATH + ".tmp%d" % os.getpid()])
        _run_all(links, verbose)
        for path in (LIB_PATH, DEBUG_LIB_PATH, PROBE_LIB_PATH):
            os.replace(path + ".tmp%d" % os.getpid(), path)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
