"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The argument validation and dispatch of libattn.so (host side of every .hip
file, instrumented by clang's sanitizers) runs the host-only ABI tests, and
the cache-blocked CPU library (instrumented by gcc's) runs its tests, each in
a subprocess with its sanitizer runtime preloaded.  A sanitizer report fails
the subprocess.  The device code is compiled as usual and never launched here.
"""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

RUN = """
import sys
sys.path.insert(0, {root!r})
import {module} as M
M.{var} = {lib!r}
import pytest
rc = pytest.main(["-q", "-p", "no:cacheprovider", {test!r}])
maps = open("/proc/self/maps").read()
if {lib!r} not in maps:
    print("sanitized library not loaded", flush=True)
    rc = 3
sys.exit(rc)
"""


def _run(module, var, lib, test, preload):
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = RUN.format(root=ROOT, module=module, var=var, lib=lib, test=os.path.join(ROOT, "tests", test))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    return r.stdout


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    if not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    from exact_io_aware_05_amd import build as B

    return B.build_sanitized(str(tmp_path_factory.mktemp("san")))


def test_host_validation_under_clang_sanitizers(sanitized):
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("clang ASan runtime not found")
    out = _run("exact_io_aware_05_amd", "LIB_PATH", sanitized[0], "test_abi_host.py", rt[-1])
    assert "passed" in out


def test_cpu_library_under_gcc_sanitizers(sanitized):
    rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(rt):
        pytest.skip("gcc ASan runtime not found")
    out = _run("exact_io_aware_05_amd.cpu", "CPU_LIB_PATH", sanitized[1], "test_cpu_flash.py", rt)
    assert "passed" in out
