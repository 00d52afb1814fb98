"""Builds libmla_verify.so (gfx950) in-tree with hipcc.

Usage: python -m speculative_decoding_mla_amd.build
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_DIR = os.path.join(PKG_DIR, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libmla_verify.so")
PEAKS_PATH = os.path.join(LIB_DIR, "mla_peaks")  # measured roofline denominators
INCLUDE = os.path.join(ROOT, "include")
SOURCES = ["mla_verify_kernels.hip", "mla_verify_api.cpp", "mla_verify_noalloc.hip", "mla_spec_ops.hip",
           "mla_spec_ops_api.cpp"]
ARCH = "gfx950"

# Every HIP translation unit: packed-fp32 VALU forms are kept out of the code.
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-inline-asm",  # m0 is named as clobbered by the LDS-DMA asm on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the gfx950 library cannot be built")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if ln.strip() and noise not in ln
            and "(ignoring feature)" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950: the shared library and the peak
    microbenchmark executable. Always recompiles (the translation units in
    parallel, then one link). Returns the library path."""
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(LIB_DIR, exist_ok=True)
    obj_dir = os.path.join(LIB_DIR, "obj")
    os.makedirs(obj_dir, exist_ok=True)
    objs = [os.path.join(obj_dir, s + ".o") for s in SOURCES]
    peaks_tmp = PEAKS_PATH + ".tmp"
    jobs = [[hipcc(), *HIP_FLAGS, "-c", "-x", "hip", "-o", o, os.path.join(CSRC, s)] for s, o in zip(SOURCES, objs)]
    jobs.append([hipcc(), *[f for f in HIP_FLAGS if f != "-fvisibility=hidden"], "-o", peaks_tmp,
                 os.path.join(CSRC, "mla_peaks.hip")])
    with ThreadPoolExecutor(max_workers=len(jobs)) as pool:
        for f in [pool.submit(_run, cmd, verbose) for cmd in jobs]:
            f.result()
    tmp = LIB_PATH + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-fPIC", "-shared", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB_PATH)
    os.replace(peaks_tmp, PEAKS_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
