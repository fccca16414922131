"""Build libplx.so for gfx950 with hipcc (in-tree, no JIT cache).

Usage: python -m parallax_local_linear_plx_amd.build [--resource-usage]
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libplx.so")
# measured ceilings (matrix-core and HBM read rate) for the benchmark; not
# part of the operator's library
PEAK_LIB = os.path.join(PKG, "libplx_peak.so")

SOURCES = ["plx_api.cpp", "plx_fwd.hip", "plx_decode.hip", "plx_bwd.hip", "plx_proj.hip"]
PEAK_SOURCES = ["plx_peak.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 VALU forms are kept off: hipcc is left to emit scalar fp32 ops.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]
# Device-side code generation: MFMA accumulators in the VGPR form.  The kernels
# rescale and read their accumulators on the VALU; with the AGPR form the
# register allocator shuttles every accumulator between the two files on each
# loop iteration (hundreds of v_accvgpr moves per 64-key tile).
DEVICE = ["-mllvm", "-amdgpu-mfma-vgpr-form"]


def _compile(src: str, resource_usage: bool) -> tuple[str, str]:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE, "-c", path, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, *COMMON, "-x", "hip", "-c", path, "-o", obj]
    if resource_usage and src.endswith(".hip"):
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    res = subprocess.run(cmd, capture_output=True, text=True)
    log = res.stdout + res.stderr
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{log}")
    return obj, log


def build(resource_usage: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES) + len(PEAK_SOURCES)) as ex:
        results = list(ex.map(lambda s: _compile(s, resource_usage), SOURCES + PEAK_SOURCES))
    peak_objs = [r[0] for r in results[len(SOURCES):]]
    results = results[:len(SOURCES)]
    objs = [r[0] for r in results]
    if resource_usage or verbose:
        for src, (_, log) in zip(SOURCES, results):
            lines = [ln for ln in log.splitlines() if "remark" in ln or "error" in ln]
            if lines:
                print(f"== {src}")
                print("\n".join(lines))
    for lib, lib_objs in ((LIB, objs), (PEAK_LIB, peak_objs)):
        tmp = lib + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *lib_objs]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(resource_usage="--resource-usage" in sys.argv, verbose=True))
