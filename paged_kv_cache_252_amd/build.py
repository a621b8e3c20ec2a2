"""Build libpagedkv.so for gfx950 with hipcc (in-tree, next to this file).

    python -m paged_kv_cache_252_amd.build          # or build() from Python

Cross-compiles without a GPU.  Every HIP source gets the packed-fp32
feature switched off for the device code; the host pass warns that it does
not know the feature, which is harmless.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libpagedkv.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")

SOURCES = ["pa_abi.cpp", "pa_decode.hip", "pa_prefill.hip", "pa_cache_ops.hip", "pa_blocks.cpp"]

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    # keep MFMA accumulators in ordinary VGPRs: the online softmax rescales
    # them with VALU ops every block, which AGPRs would force through copies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libpagedkv")


def build(verbose: bool = False, save_temps: str | None = None) -> str:
    """Compile every source into ``libpagedkv.so``; returns its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *FLAGS, "-shared", "-I", INCLUDE, "-I", CSRC]
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        cmd += ["--save-temps"]          # intermediate files land in save_temps (the cwd)
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        cmd += (["-x", "hip", path] if src.endswith(".cpp") else [path])
    cmd += ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=save_temps or HERE, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
