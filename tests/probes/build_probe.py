"""Build the probe libraries next to this file (hipcc, gfx950): libexp2_probe.so (the tests'
hardware-exp2 check), libhbm_ceiling.so (the bench's read and copy ceilings),
libmfma_ceiling.so (the bench's dense BF16 matrix-core ceiling) and liblds_ceiling.so (the LDS
read and direct-to-LDS load rates per CU)."""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from deterministic_selected_token_amd import build as lib_build  # noqa: E402

PROBES = {"libexp2_probe.so": "exp2_probe.hip", "libhbm_ceiling.so": "hbm_ceiling.hip",
          "libmfma_ceiling.so": "mfma_ceiling.hip", "liblds_ceiling.so": "lds_ceiling.hip"}
OUT = os.path.join(HERE, "libexp2_probe.so")
CEILING = os.path.join(HERE, "libhbm_ceiling.so")
MFMA_CEILING = os.path.join(HERE, "libmfma_ceiling.so")


def build() -> list[str]:
    flags = [f for f in lib_build.HIPCC_FLAGS if f != "-fvisibility=hidden"]
    built = []
    for lib, src in PROBES.items():
        out = os.path.join(HERE, lib)
        tmp = out + f".tmp{os.getpid()}"
        subprocess.run([lib_build.hipcc(), *flags, "-o", tmp, os.path.join(HERE, src)],
                       check=True)
        os.replace(tmp, out)
        built.append(out)
    return built


if __name__ == "__main__":
    print("\n".join(build()))
