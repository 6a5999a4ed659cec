"""Helpers for the GPU parity tests: upload seeded inputs, compare with the oracle.

Tolerances (applied per output tensor, or per sampled subset of it):
* float32 inputs: max |gpu - oracle| <= 1e-5;
* bfloat16 outputs and gradients: max |gpu - oracle| <= 2e-2 and
  ||gpu - oracle||_F / ||oracle||_F <= 1e-2.
LSE is float32 in both paths and is held to the same rule as its inputs' dtype.
"""

import numpy as np
import pytest
import torch

F32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_REL_FRO = 1e-2


def have_gpu():
    return torch.cuda.is_available()


def upload(raw, dtype, device="cuda"):
    """numpy raw array (uint16 bf16 bits or float32) -> torch tensor on the GPU."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(raw, dtype=np.float32))
    return t.to(device)


def download(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = gpu - ref
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(d) / nref) if nref > 0 else float(np.linalg.norm(d))
    return max_abs, rel


def assert_close(gpu, ref, dtype, what=""):
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    max_abs, rel = errors(gpu, ref)
    if dtype == "fp32":
        assert max_abs <= F32_MAX_ABS, f"{what}: max abs {max_abs:.3e} > {F32_MAX_ABS}"
    else:
        assert max_abs <= BF16_MAX_ABS, f"{what}: max abs {max_abs:.3e} > {BF16_MAX_ABS}"
        assert rel <= BF16_REL_FRO, f"{what}: rel Frobenius {rel:.3e} > {BF16_REL_FRO}"
    return max_abs, rel


gpu = pytest.mark.gpu
needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def oracle_map(fn, items):
    """Run an oracle function over independent items (usually heads) on the
    host cores: a thread pool of up to 16 workers, one BLAS thread each
    (numpy releases the GIL inside its kernels).  Results in item order."""
    import concurrent.futures
    import os

    from threadpoolctl import threadpool_limits

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with threadpool_limits(1):
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            return list(ex.map(fn, items))
