"""The diagnostic microbenchmark library (libattn_probe.so): it loads and
exports its entry points, rejects bad sizes on the host, and (on a GPU) its
atomic-add probe ends with exact counts and its timing probes return sane
figures."""

import ctypes
import os

import pytest

from exact_io_aware_05_amd import diag


def test_probe_library_exports():
    L = diag.lib()
    for name in ("probe_atomic_dq", "probe_issue_mix", "probe_mfma_rate", "probe_read_bw"):
        assert hasattr(L, name), name


def test_probe_rejects_bad_sizes_on_the_host():
    L = diag.lib()
    ms, bad = ctypes.c_float(), ctypes.c_longlong()
    assert L.probe_atomic_dq(64, 7, 256, 0, 1, 1, ctypes.byref(ms), ctypes.byref(bad)) != 0  # heads % 8
    assert L.probe_atomic_dq(64, 8, 200, 0, 1, 1, ctypes.byref(ms), ctypes.byref(bad)) != 0  # n % 128
    assert L.probe_atomic_dq(96, 8, 256, 0, 1, 1, ctypes.byref(ms), ctypes.byref(bad)) != 0  # d
    mean, mx = ctypes.c_double(), ctypes.c_double()
    assert L.probe_issue_mix(10, 1, 256, ctypes.byref(mean), ctypes.byref(mx)) != 0
    assert L.probe_issue_mix(0, 3, 256, ctypes.byref(mean), ctypes.byref(mx)) != 0
    tf, ghz = ctypes.c_double(), ctypes.c_double()
    assert L.probe_mfma_rate(0, 10, ctypes.byref(tf), ctypes.byref(ghz)) != 0
    assert L.probe_read_bw(1000, 8, 8, 1, ctypes.byref(ms)) != 0  # not a multiple of 16
    assert L.probe_read_bw(1 << 20, 8, 5, 1, ctypes.byref(ms)) != 0  # unroll
    assert L.probe_read_bw(1 << 20, 0, 8, 1, ctypes.byref(ms)) != 0  # grid


@pytest.fixture(scope="module")
def cus():
    import torch

    return torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.gpu
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_atomic_probe_counts_are_exact(cus, d, causal):
    print(f"atomic probe d={d} causal={causal}", flush=True)
    for atomic in (True, False):
        r = diag.atomic_dq(d, 8, 256, causal, atomic, reps=3)
        assert r["mismatches"] == 0
        assert r["ms"] > 0


@pytest.mark.gpu
def test_issue_and_rate_probes(cus):
    r = diag.issue_mix(0, 1, cus)  # 16 MFMA of 32 cycles each
    assert 400 < r["max_cycles"] < 800
    r = diag.mfma_rate(cus, iters=2000)
    assert r["tflops"] > 0 and 0.5 < r["ghz"] < 4.0
    r = diag.read_bw(64 << 20, 4 * cus, reps=3)
    assert r["ms"] > 0 and r["GB_per_s"] < 8000 * 1.05


def test_bindings_load_torch_before_their_hip_library():
    """Both ctypes bindings import torch before loading a HIP library, so the
    library binds to torch's HIP runtime (same soname) instead of loading the
    system runtime beside it, which would see no GPU once torch's holds it."""
    import subprocess
    import sys

    code = (
        "import sys\n"
        "import exact_io_aware_05_amd as E\n"
        "from exact_io_aware_05_amd import diag\n"
        "assert 'torch' not in sys.modules\n"
        "E.lib()\n"
        "assert 'torch' in sys.modules\n"
        "diag.lib()\n"
        "print('ok')\n"
    )
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stderr[-2000:]
