"""Build libq4moe.so (HIP, gfx950) in-tree with hipcc.

Every ``csrc/*.hip`` file is compiled to an object under ``_build/`` (in
parallel), then linked into ``quantized_moe_decode_affine_amd/libq4moe.so``.
Always recompiles; run ``python -m quantized_moe_decode_affine_amd.build``.

``--stamps`` also links ``libq4moe_stamps.so``: the same library with the decode
layer kernel built with phase stamps (``-DQ4MOE_DECODE_STAMPS``) and the grouped
GEMM with workgroup stamps (``-DQ4MOE_GEMM_STAMPS``), read by ``phase_timeline.py``.
The product path never loads it.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libq4moe.so")
STAMPS_LIB = os.path.join(PKG, "libq4moe_stamps.so")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Wno-unused-command-line-argument",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in ordinary VGPRs (the per-group scale fold reads them with VALU ops)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # single-lane atomics stay single atomics (the optimizer's lane aggregation reads the
    # result back at once, which makes a wave wait for a counter it needs only later)
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-I" + os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libq4moe")


def _run(cmd):
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in proc.stderr.splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"build step failed ({proc.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in sources]
    with ThreadPoolExecutor(min(8, len(sources))) as pool:
        logs = list(pool.map(lambda so: _run([hipcc, *CFLAGS, "-c", so[0], "-o", so[1]]), zip(sources, objs)))
    if verbose:
        for s, log in zip(sources, logs):
            if log.strip():
                print(f"[{os.path.basename(s)}]\n{log}")
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


# sources rebuilt with stamps in the diagnostic library, and their macros
STAMPED = {"decode.hip": "-DQ4MOE_DECODE_STAMPS", "decode_batch.hip": "-DQ4MOE_DECODE_STAMPS",
           "gemm.hip": "-DQ4MOE_GEMM_STAMPS"}


def build_stamps() -> str:
    """The diagnostic library: every object of build(), the decode layer kernels (batch-1
    and the batched front launch) and the grouped GEMM rebuilt with stamps."""
    hipcc = _hipcc()
    build()
    d = os.path.join(BUILD, "stamps")
    os.makedirs(d, exist_ok=True)
    stamped = []
    for src, flag in STAMPED.items():
        obj = os.path.join(d, src[:-4] + ".o")
        _run([hipcc, *CFLAGS, flag, "-c", os.path.join(CSRC, src), "-o", obj])
        stamped.append(obj)
    skip = {src[:-4] + ".o" for src in STAMPED}
    objs = [o for o in sorted(glob.glob(os.path.join(BUILD, "*.o"))) if os.path.basename(o) not in skip]
    tmp = STAMPS_LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, *stamped, "-o", tmp])
    os.replace(tmp, STAMPS_LIB)
    return STAMPS_LIB


if __name__ == "__main__":
    print(build_stamps() if "--stamps" in sys.argv else build(verbose="-v" in sys.argv))
