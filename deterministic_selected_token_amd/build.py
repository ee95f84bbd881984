"""Build the gfx950 C-ABI library ``liblogp_mi355x.so`` in-tree with hipcc."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "liblogp_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = [os.path.join(CSRC, f) for f in ("logp_kernels.hip", "grpo_kernels.hip",
                                            "linear_kernels.hip")]
HEADERS = [os.path.join(CSRC, "logp_device.hpp"), os.path.join(CSRC, "host_common.hpp"),
           os.path.join(INCLUDE, "logp.h"), os.path.join(INCLUDE, "grpo_loss.h"),
           os.path.join(INCLUDE, "linear_logp.h")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-mcode-object-version=5",    # also loadable by the ROCm 7.0 runtime bundled with torch
    "-ffp-contract=off",          # no implicit FMA: every kernel rounds the same way
    "-fno-fast-math",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
    "-Wall",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: cannot build the gfx950 library")


def command(out: str = LIB_PATH, extra: list[str] | None = None) -> list[str]:
    return [hipcc(), *HIPCC_FLAGS, *(extra or []), f"-I{INCLUDE}", f"-I{CSRC}", "-o", out,
            *SOURCES]


def stale() -> bool:
    if not os.path.exists(LIB_PATH):
        return True
    t = os.path.getmtime(LIB_PATH)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


def build(verbose: bool = False) -> str:
    """Compile every source; always rebuilds (the build check compiles each time)."""
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB_PATH)
