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
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    # only the explicit fmaf() calls fuse: the sums have one fixed rounding order
    "-ffp-contract=off",
    # keep the compiler from forming packed fp32 ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, *(extra or []), "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
