"""Build libattn.so (the C ABI plus every HIP kernel) for gfx950 with hipcc.

The library is built in-tree, next to this file, so that it travels with the
source tree.  Every source is compiled to its own object (in parallel, under
_build/ at the repository root) and the objects are linked into the library,
so that a source can carry device-compiler flags of its own (PER_FILE).
Packed-fp32 instructions are disabled in device code
(-target-feature -packed-fp32-ops); hipcc's host pass warns that it does not
know the feature, which is harmless.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libattn.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "--offload-arch=gfx950"
FLAGS = [
    ARCH, "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]
# Extra device-compiler flags per source file.
PER_FILE = {
    # MFMA accumulators in ordinary VGPRs: otherwise the compiler copies the
    # loop-carried dQ blocks to AGPRs and back in every iteration.
    "bwd_dq.hip": ["-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form"],
    # the same for the D = 512 kernel: its online-softmax rescale of the O
    # accumulator otherwise runs on AGPR copies
    "fwd_d512.hip": ["-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form"],
}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(
        glob.glob(os.path.join(CSRC, "*.cpp")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    return subprocess.run(cmd, capture_output=True, text=True)


def build(verbose: bool = False) -> str:
    """Compile every HIP source and the C ABI into libattn.so (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = []
    for src in sources():
        name = os.path.basename(src)
        obj = os.path.join(BUILD_DIR, name + ".o")
        jobs.append((obj, [HIPCC, *FLAGS, *PER_FILE.get(name, []), "-c", src, "-o", obj]))
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as pool:
        results = list(pool.map(lambda j: _run(j[1], verbose), jobs))
    failed = [r for r in results if r.returncode != 0]
    if failed:
        for r in failed:
            sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed to compile a source of libattn.so")
    tmp = LIB_PATH + ".tmp"
    res = _run([HIPCC, ARCH, "-shared", "-fPIC", *[obj for obj, _ in jobs], "-o", tmp], verbose)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to link libattn.so")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
