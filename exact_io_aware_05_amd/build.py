"""Build the HIP attention library (``libattn.so``) for gfx950 with hipcc, the
CPU library (``libattn_cpu.so``) with g++, and the diagnostic microbenchmarks
(``libattn_probe.so``, not part of the attention library).

Run as ``python -m exact_io_aware_05_amd.build``.  Each ``csrc/*.hip`` file is
compiled to an object in ``_build/`` (in parallel), then linked in-tree to
``exact_io_aware_05_amd/libattn.so``; ``csrc/attn_cpu.cpp`` becomes
``exact_io_aware_05_amd/libattn_cpu.so`` and ``probe/attn_probe.hip``
``exact_io_aware_05_amd/libattn_probe.so``.
"""

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattn.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 VALU instructions are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-I",
    os.path.join(ROOT, "include"),
] + DEVICE_FLAGS


CPU_LIB = os.path.join(PKG, "libattn_cpu.so")
CXX = os.environ.get("CXX", "g++")
# The CPU library (include/attn_cpu.h): AVX2 + FMA, which every x86-64 host of
# an MI355X supports, and OpenMP.
CPU_FLAGS = ["-O3", "-mavx2", "-mfma", "-fopenmp", "-fPIC", "-shared", "-std=c++17", "-Wall", "-Wextra"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build_cpu():
    """Compile csrc/attn_cpu.cpp into exact_io_aware_05_amd/libattn_cpu.so."""
    tmp = CPU_LIB + ".tmp"
    cmd = [CXX] + CPU_FLAGS + ["-I", os.path.join(ROOT, "include"), os.path.join(CSRC, "attn_cpu.cpp"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"g++ failed for attn_cpu.cpp:\n{r.stderr}")
    os.replace(tmp, CPU_LIB)
    return CPU_LIB


PROBE_LIB = os.path.join(PKG, "libattn_probe.so")


def build_probe():
    """Compile probe/attn_probe.hip into exact_io_aware_05_amd/libattn_probe.so."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, os.path.join(PKG, "probe", "attn_probe.hip"), "-shared", "-o", tmp] + COMMON
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        err = "\n".join(line for line in (r.stderr or "").splitlines() if "packed-fp32-ops" not in line)
        raise RuntimeError(f"hipcc failed for attn_probe.hip:\n{err}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, "-c", src, "-o", obj] + COMMON
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(
        line for line in (r.stderr or "").splitlines() if "packed-fp32-ops" not in line
    )
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj, err


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    for obj, err in results:
        if verbose and err.strip():
            print(err)
    objs = [o for o, _ in results]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-o", tmp] + objs + [f"--offload-arch={ARCH}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    build_cpu()
    build_probe()
    return LIB


# Host-side sanitizer flags for hipcc: each -fsanitize= behind -Xarch_host, so
# only the host code (argument validation, dispatch) is instrumented and the
# device code is compiled as usual.
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer"]


def build_sanitized(dest):
    """AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code, for
    checks on a CPU: ``dest/libattn_san.so`` (every csrc/*.hip file, host side
    instrumented by clang's sanitizers; run under clang's ASan runtime) and
    ``dest/libattn_cpu_san.so`` (attn_cpu.cpp under gcc's sanitizers; run under
    gcc's libasan).  Returns the two paths."""
    os.makedirs(dest, exist_ok=True)
    objdir = os.path.join(dest, "obj")
    os.makedirs(objdir, exist_ok=True)
    flags = [f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include")]
    flags += DEVICE_FLAGS + SAN_HOST

    def comp(src):
        obj = os.path.join(objdir, os.path.basename(src)[:-4] + ".o")
        r = subprocess.run([HIPCC, "-c", src, "-o", obj] + flags, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc (sanitized) failed for {src}:\n{r.stderr}")
        return obj

    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(comp, srcs))
    hip_lib = os.path.join(dest, "libattn_san.so")
    r = subprocess.run([HIPCC, "-shared", "-o", hip_lib] + objs + [f"--offload-arch={ARCH}"] + SAN_HOST
                       + ["-Xarch_host", "-shared-libsan"], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (sanitized) failed:\n{r.stderr}")
    cpu_lib = os.path.join(dest, "libattn_cpu_san.so")
    cmd = [CXX, "-O1", "-g", "-mavx2", "-mfma", "-fopenmp", "-fPIC", "-shared", "-std=c++17",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), os.path.join(CSRC, "attn_cpu.cpp"), "-o", cpu_lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"g++ (sanitized) failed:\n{r.stderr}")
    return hip_lib, cpu_lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
