"""O(N) memory of the fused path (the point of the method: the N x N score and
probability matrices are never stored; "Memory" / "Key Ideas" on the Paper
Notes page, "The backward pass: recompute instead of store" on the aicassindra
page).

Forward + backward at B=1, H=8, d=64, causal, N in {16K, 32K, 64K} (the
largest is the long-context workload): device memory beyond the inputs must be
exactly the outputs (O, LSE, dQ, dK, dV) plus the backward workspace (D), all
linear in N, and the library itself must allocate nothing (free device memory
drops by no more than what torch's caching allocator reserved).  One head's
bf16 score matrix alone would be 8 GiB at N = 64K.
"""

import pytest
import torch

pytestmark = [pytest.mark.gpu]

B, H, D = 1, 8, 64
SLACK = 1 << 20  # allocator rounding (512-byte blocks, small-pool segments)
RUNTIME_SLACK = 4 << 20  # HIP runtime bookkeeping; any N x N buffer is >= 512 MiB here


def _api():
    import exact_io_aware_05_amd as E

    E.lib()
    return E


def _extra_bytes(n):
    """Peak bytes allocated beyond the inputs during fwd + bwd, and the bytes
    the outputs and workspace account for."""
    E = _api()
    print(f"[case] memory B={B} H={H} N={n} d={D} causal", flush=True)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    g = torch.Generator(device="cuda").manual_seed(5)
    q, k, v, do = (torch.randn(B, H, n, D, device="cuda", generator=g).to(torch.bfloat16) for _ in range(4))
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    reserved0 = torch.cuda.memory_reserved()
    free0, _ = torch.cuda.mem_get_info()
    o, lse = E.attn_fwd(q, k, v, causal=True)
    dq, dk, dv = E.attn_bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    # The peak can be no lower than what is still allocated (the outputs); a
    # peak statistic read below that (seen once, 0 bytes) falls back to it.
    peak = max(torch.cuda.max_memory_allocated(), torch.cuda.memory_allocated()) - base
    free1, _ = torch.cuda.mem_get_info()
    reserved1 = torch.cuda.memory_reserved()
    tensor_bytes = 4 * B * H * n * D * 2 + B * H * n * 4  # O, dQ, dK, dV (bf16) + LSE (fp32)
    workspace = E.attn_bwd_workspace_bytes(B, H, n, D, E.ATTN_BF16)
    assert bool(torch.isfinite(dq.float()).all()) and bool(torch.isfinite(dv.float()).all())
    # Whatever the device lost that torch did not reserve was allocated elsewhere.
    outside_torch = (free0 - free1) - (reserved1 - reserved0)
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    return peak, tensor_bytes, workspace, outside_torch


def test_memory_is_linear_in_n_and_library_allocates_nothing():
    # Load the kernels' code (first launch) before measuring device memory.
    _extra_bytes(256)
    peaks = {}
    for n in (16384, 32768, 65536):
        peak, tensor_bytes, workspace, outside = _extra_bytes(n)
        print(f"N={n}: peak extra {peak} B, outputs {tensor_bytes} B, workspace {workspace} B, "
              f"outside torch {outside} B", flush=True)
        assert workspace == B * H * n * 4 or workspace == ((B * H * n * 4 + 255) // 256) * 256
        assert peak <= tensor_bytes + workspace + SLACK, (n, peak, tensor_bytes, workspace)
        assert outside <= RUNTIME_SLACK, (n, outside)
        # Nothing quadratic: less than a quarter of one head's bf16 score
        # matrix (2 N^2 bytes).
        assert peak < n * n // 2
        peaks[n] = peak
    # Doubling N doubles the extra memory (within the slack), never quadruples it.
    for a, b in ((16384, 32768), (32768, 65536)):
        assert abs(peaks[b] - 2 * peaks[a]) <= 4 * SLACK, (a, b, peaks)
