"""Compile libzs.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

The library is built in-tree next to this file.  Compiler flags that matter
for results:

* ``-ffp-contract=off``: fp32 multiplies and adds stay separately rounded, as
  in the materialised-message reference; the fp64 channel sums use explicit
  ``fma`` calls, which this flag does not affect.
* ``-fno-gpu-flush-denormals-to-zero``: fp32 subnormals are kept (IEEE).
* ``-Xclang -target-feature -Xclang -packed-fp32-ops``: no packed fp32 VALU
  instructions are generated.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libzs.so")
SOURCES = ["zs_api.hip", "zs_csr.hip", "zs_fwd.hip", "zs_bwd.hip", "zs_norm.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def build(verbose: bool = False) -> str:
    """Compile every source into libzs.so (always recompiles)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


def device_asm(out_dir: str) -> list[str]:
    """Write the gfx950 assembly of every kernel source (for instruction checks)."""
    os.makedirs(out_dir, exist_ok=True)
    paths = []
    for s in SOURCES:
        out = os.path.join(out_dir, s.replace(".hip", f"-{ARCH}.s"))
        subprocess.check_call([HIPCC, *[f for f in FLAGS if f not in ("-shared", "-fPIC")],
                               "--cuda-device-only", "-S", os.path.join(CSRC, s), "-o", out])
        paths.append(out)
    return paths


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
