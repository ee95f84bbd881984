"""Build the test probe library tests/probes/libexp2_probe.so (hipcc, gfx950)."""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from deterministic_selected_token_amd import build as lib_build  # noqa: E402

SRC = os.path.join(HERE, "exp2_probe.hip")
OUT = os.path.join(HERE, "libexp2_probe.so")


def build() -> str:
    flags = [f for f in lib_build.HIPCC_FLAGS if f != "-fvisibility=hidden"]
    tmp = OUT + f".tmp{os.getpid()}"
    subprocess.run([lib_build.hipcc(), *flags, "-o", tmp, SRC], check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
