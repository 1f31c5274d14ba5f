"""Build libpa.so (the gfx950 kernels + C ABI) in-tree with hipcc.

    python -m paged_quantized_kv_reshape_amd.build            # release build
    PA_HIPCC_FLAGS="-save-temps" python -m ...build            # extra flags

hipcc cross-compiles for gfx950 without a GPU present.
"""
from __future__ import annotations

import os
import shlex
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpa.so")
SOURCES = ["pa_api.cpp", "pa_alloc.cpp", "pa_write.hip", "pa_decode.hip", "pa_merge.hip",
           "pa_blocks.hip", "pa_prefill.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    # IEEE fp32 division and sqrt: the quantizers divide by their scale and the outlier
    # statistics take square roots, both correctly rounded.
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *shlex.split(os.environ.get("PA_HIPCC_FLAGS", "")), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(shlex.quote(c) for c in cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout or "") + (r.stderr or "")
    # the host pass does not know the packed-fp32 target feature; that warning is expected
    noise = "is not a recognized feature for this target"
    lines = [ln for ln in out.splitlines() if noise not in ln and "(ignoring feature)" not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
