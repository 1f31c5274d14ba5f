"""The host code of libpa under the compiler's sanitizers, on the CPU.

* AddressSanitizer + UndefinedBehaviorSanitizer (any report aborts): the C ABI's argument
  checks (pa_api.cpp) and the block allocator (pa_alloc.cpp), built with g++ into a shared
  library whose kernel launchers are stand-ins (tests/sanitize/launch_stubs.cpp), driven by
  the ABI and allocator tests and by well-formed calls that pass every check
  (tests/sanitize/abi_valid_calls.py).
* ThreadSanitizer: eight threads allocating, sharing, copying on write and releasing blocks
  of one allocator at once (tests/sanitize/alloc_threads.cpp).

The pages' failure mode for this path is an illegal memory access (xonoai.com report on
vLLM v0.7.2, "Deconstructing the v0.7.2 Architecture"); the device side guards against it
with its own checks, and these runs cover the host side."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_quantized_kv_reshape_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"{name} not available")
    return path


def test_abi_and_allocator_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    lib = tmp_path / "libpa_asan.so"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), os.path.join(CSRC, "pa_api.cpp"),
           os.path.join(CSRC, "pa_alloc.cpp"), os.path.join(SAN, "launch_stubs.cpp"),
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", str(lib)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    driver = (
        "import sys\n"
        f"sys.path.insert(0, {ROOT!r}); sys.path.insert(0, {os.path.join(ROOT, 'tests')!r})\n"
        "import paged_quantized_kv_reshape_amd.binding as B\n"
        f"B._LIB_PATH = {str(lib)!r}\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider',\n"
        f"    {os.path.join(ROOT, 'tests', 'test_abi.py')!r},\n"
        f"    {os.path.join(ROOT, 'tests', 'test_allocator.py')!r},\n"
        f"    {os.path.join(SAN, 'abi_valid_calls.py')!r},\n"
        "    '-k', 'not exports_every and not environment_knob and not static_scratch']))\n")
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", driver], capture_output=True, text=True, env=env,
                       timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail


def test_allocator_threads_under_tsan(tmp_path):
    _runtime("libtsan.so")
    exe = tmp_path / "alloc_tsan"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=thread",
           "-I" + os.path.join(ROOT, "include"), os.path.join(SAN, "alloc_threads.cpp"),
           os.path.join(CSRC, "pa_alloc.cpp"), "-lpthread", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, TSAN_OPTIONS="halt_on_error=1"))
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "alloc_threads ok" in r.stdout
    assert "WARNING: ThreadSanitizer" not in r.stderr
