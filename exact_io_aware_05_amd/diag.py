"""ctypes binding of ``libattn_probe.so``: diagnostic microbenchmarks on gfx950
(``probe/attn_probe.hip``), separate from the attention library.  They measure
facts the kernels' design rests on: the throughput of fp32 atomic adds for a
dQ accumulated by key blocks, how much vector work hides under the matrix
instructions of one wave, and the MFMA rate and shader clock under load.
``python bench.py --probes`` runs them all.
"""

import ctypes
import os

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn_probe.so")
_lib = None

MIXES = {
    0: "16 MFMA",
    1: "16 x (MFMA, 4 FMA)",
    2: "16 x (MFMA, 6 FMA)",
    3: "16 x (MFMA, 7 FMA)",
    4: "16 x (MFMA, 8 FMA)",
    5: "16 x (MFMA, exp, 3 FMA)",
    6: "16 MFMA, then 64 FMA",
    7: "64 FMA",
    8: "64 exp",
    9: "16 x (MFMA, LDS read, 4 FMA, wait for the read)",
}


def _bind_torch_runtime():
    """torch ships its own HIP runtime under the system's soname: loading torch
    first makes this library bind to that one runtime (a second copy loaded
    beside it sees no GPU once the first holds it)."""
    try:
        import torch  # noqa: F401
    except ImportError:
        pass


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_PATH):
            raise RuntimeError(f"{_PATH} is not built: run python -m exact_io_aware_05_amd.build")
        _bind_torch_runtime()
        L = ctypes.CDLL(_PATH)
        i = ctypes.c_int
        L.probe_atomic_dq.argtypes = [i, i, i, i, i, i, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_longlong)]
        L.probe_issue_mix.argtypes = [i, i, i, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
        L.probe_mfma_rate.argtypes = [i, i, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
        L.probe_read_bw.argtypes = [ctypes.c_longlong, i, i, i, ctypes.POINTER(ctypes.c_float)]
        for f in (L.probe_atomic_dq, L.probe_issue_mix, L.probe_mfma_rate, L.probe_read_bw):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with HIP error {rc}")


def atomic_dq(d, heads, n, causal, atomic, reps=10):
    """fp32 atomic adds (atomic=True) or plain stores of the dQ tiles a
    key-block pass would add: ms per launch, bytes added, GB/s, and the number
    of elements that end with the wrong value."""
    ms, bad = ctypes.c_float(), ctypes.c_longlong()
    _check(lib().probe_atomic_dq(d, heads, n, int(causal), int(atomic), reps, ctypes.byref(ms), ctypes.byref(bad)),
           "probe_atomic_dq")
    nblk, ntile = n // 128, n // 64
    tiles = sum(ntile - 2 * b if causal else ntile for b in range(nblk)) * heads
    nbytes = tiles * 64 * d * 4
    return {"ms": ms.value, "bytes": nbytes, "GB_per_s": nbytes / (ms.value * 1e-3) / 1e9, "mismatches": bad.value}


def issue_mix(mix, waves_per_simd, num_cus):
    """Cycles per iteration of instruction mix ``mix`` (see MIXES): mean over
    the waves and the largest."""
    mean, mx = ctypes.c_double(), ctypes.c_double()
    _check(lib().probe_issue_mix(mix, waves_per_simd, num_cus, ctypes.byref(mean), ctypes.byref(mx)), "probe_issue_mix")
    return {"mean_cycles": mean.value, "max_cycles": mx.value}


def mfma_rate(num_cus, iters=20000):
    """Back-to-back bf16 MFMAs on every SIMD: TFLOP/s and shader clock (GHz)."""
    tf, ghz = ctypes.c_double(), ctypes.c_double()
    _check(lib().probe_mfma_rate(num_cus, iters, ctypes.byref(tf), ctypes.byref(ghz)), "probe_mfma_rate")
    return {"tflops": tf.value, "ghz": ghz.value}


def read_bw(nbytes, grid, unroll=8, reps=20):
    """Plain streaming read of ``nbytes`` by ``grid`` workgroups: ms per
    launch and GB/s."""
    ms = ctypes.c_float()
    _check(lib().probe_read_bw(nbytes, grid, unroll, reps, ctypes.byref(ms)), "probe_read_bw")
    return {"ms": ms.value, "GB_per_s": nbytes / (ms.value * 1e-3) / 1e9}

