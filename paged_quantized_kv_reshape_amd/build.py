"""Build libpa.so (the gfx950 kernels + C ABI) in-tree with hipcc.

    python -m paged_quantized_kv_reshape_amd.build            # release build
    PA_HIPCC_FLAGS="-save-temps" python -m ...build            # extra flags

Each source compiles to its own object under _build/ (in parallel), then hipcc links the
shared library. hipcc cross-compiles for gfx950 without a GPU present.
"""
from __future__ import annotations

import os
import shlex
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpa.so")
OBJ_DIR = os.path.join(ROOT, "_build")
SOURCES = ["pa_api.cpp", "pa_alloc.cpp", "pa_write.hip", "pa_decode.hip", "pa_merge.hip",
           "pa_blocks.hip", "pa_prefill.hip", "pa_static.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
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
# the host pass does not know the packed-fp32 target feature; that warning is expected
_NOISE = ("is not a recognized feature for this target", "(ignoring feature)")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout or "") + (r.stderr or "")
    lines = [ln for ln in out.splitlines() if not any(n in ln for n in _NOISE)]
    return r.returncode, lines


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    extra = shlex.split(os.environ.get("PA_HIPCC_FLAGS", ""))
    jobs = []
    for s in SOURCES:
        obj = os.path.join(OBJ_DIR, os.path.splitext(s)[0] + ".o")
        jobs.append((obj, [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, s), "-o", obj]))
    if verbose:
        for _, cmd in jobs:
            print(" ".join(shlex.quote(c) for c in cmd), flush=True)
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(lambda j: _run(j[1]), jobs))
    failed = [(j, lines) for j, (rc, lines) in zip(jobs, results) if rc != 0]
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(
            f"--- {os.path.basename(j[0])}\n" + "\n".join(lines) for j, lines in failed))
    if verbose:
        for lines in (ln for _, ln in results if ln):
            print("\n".join(lines))
    tmp = LIB + ".tmp"
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for o, _ in jobs], "-o", tmp]
    if verbose:
        print(" ".join(shlex.quote(c) for c in link), flush=True)
    rc, lines = _run(link)
    if rc != 0:
        raise RuntimeError("hipcc link failed:\n" + "\n".join(lines))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
