"""Build libcfm.so (the HIP library behind include/cfm.h) in-tree for gfx950.

    python calibration_free_channel_amd/build.py [-j N] [--trace]

Compiles every csrc/*.hip translation unit with hipcc and links them into
calibration_free_channel_amd/libcfm.so (with --trace: the instrumented
libcfm_trace.so, phase timestamps compiled in). Always recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcfm.so")
# instrumented build (phase timestamps, cfm_phase_trace); loaded only when
# CFM_PHASE_TRACE=1 is set in the environment
TRACE_LIB = os.path.join(PKG, "libcfm_trace.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed FP32 instructions are disabled for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, trace: bool = False) -> str:
    obj = os.path.join(BUILD + ("_trace" if trace else ""), os.path.basename(src).replace(".hip", ".o"))
    cmd = [HIPCC, *CFLAGS, *(["-DCFM_PHASE_TRACE"] if trace else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8, verbose: bool = True, trace: bool = False) -> str:
    os.makedirs(BUILD + ("_trace" if trace else ""), exist_ok=True)
    lib = TRACE_LIB if trace else LIB
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda f: _compile(f, trace), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(srcs)} sources")
    return lib


if __name__ == "__main__":
    j = int(sys.argv[sys.argv.index("-j") + 1]) if "-j" in sys.argv else 8
    build(j, trace="--trace" in sys.argv)
