"""Build libqsa.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libqsa.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
# The benchmark's gather probe: a measurement aid in a library of its own.
PROBE_LIB_PATH = os.path.join(PKG_DIR, "libqsa_probe.so")
PROBE_SOURCES = ["probe.hip"]

SOURCES = ["indexer.hip", "topk.hip", "select_fused.hip", "attention.hip", "attention_tile.hip",
           "backward.hip", "warmup.hip", "qsa_abi.hip"]

# Packed fp32 VALU ops are disabled for all device code (the hipcc host pass warns
# that it does not know the feature; that warning is harmless).
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
# Per-source device flags. attention.hip keeps its MFMA accumulators in VGPRs: with
# them in AGPRs the compiler copies all of them out and back around every step's
# conditional rescale, and needs 264 registers where the VGPR form needs 198 (two
# waves per SIMD; the decode kernels go from 304 to 180-238 registers).
SOURCE_FLAGS = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
_NOISE = "is not a recognized feature for this target"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libqsa)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if _NOISE not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)


def build_library(sources, out_path, verbose=False, extra_flags=()):
    """Compile each source to an object (in parallel), then link a shared library."""
    cc = hipcc()
    jobs = max(1, min(len(sources), int(os.environ.get("MAX_JOBS", "8"))))
    with tempfile.TemporaryDirectory(prefix="qsa_build_") as tmpd:
        objs = [os.path.join(tmpd, os.path.splitext(s)[0] + ".o") for s in sources]
        cmds = [[cc, *HIP_FLAGS, *SOURCE_FLAGS.get(s, []), *extra_flags, "-I", INCLUDE, "-I",
                 CSRC, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(sources, objs)]
        with ThreadPoolExecutor(jobs) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = out_path + ".tmp"
        _run([cc, *HIP_FLAGS, *extra_flags, "-shared", "-o", tmp, *objs], verbose)
        os.replace(tmp, out_path)
    return out_path


def build(verbose: bool = False) -> str:
    """Compile every HIP source: libqsa.so (LIB_PATH) and the benchmark's probe
    library; always rebuilds. Returns the path of libqsa.so."""
    build_library(PROBE_SOURCES, PROBE_LIB_PATH, verbose)
    return build_library(SOURCES, LIB_PATH, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
