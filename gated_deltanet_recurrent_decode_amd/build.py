"""Build libgdn.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

    python -m gated_deltanet_recurrent_decode_amd.build [-v]
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgdn.so")
SOURCES = ["gdn_abi.hip", "gdn_step.hip", "gdn_step_tile.hip", "gdn_prefill.hip", "conv_decode.hip", "slot_commit.hip", "slot_ops.hip",
           "traffic_probe.hip", "gdn_prefill_two_pass.hip"]
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # only the explicit fmaf() calls fuse: the sums have one fixed rounding order
    "-ffp-contract=off",
    # keep the compiler from forming packed fp32 ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]

# Flags of single sources.  The step kernels take what their first round of
# scalar loads needs (the tile kernel: slot arrays, gate arrays, B, H_v, G,
# the grid size; the walk kernel: the read slots, H_k, N) as leading
# arguments that the hardware preloads into scalar registers (gfx950 kernel
# argument preloading), so the slots are requested at once instead of after a
# load of the arguments.  Code objects built with preloading start with a
# block that loads the same registers, so they run unchanged where the
# firmware does not preload.
PER_SOURCE = {
    "gdn_step_tile.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=8"],
    "gdn_step.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=3"],
    # the calibration copies, so that their slot loads leave as early as the step's
    "traffic_probe.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=9"],
}


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile each source to an object (in parallel), then link them."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [hipcc(), *FLAGS, *PER_SOURCE.get(src, []), *(extra or []), "-I", INCLUDE, "-I", CSRC, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((src, obj, subprocess.Popen(cmd)))
    failed = [src for src, _, pr in jobs if pr.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, "hipcc " + " ".join(failed))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *[obj for _, obj, _ in jobs], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
