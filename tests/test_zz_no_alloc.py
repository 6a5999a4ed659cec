"""attn_bwd_noalloc (no allocation, fixed device scratch) against attn_bwd.

Both entry points run the same kernels; the allocation-free one keeps D in the
library's fixed device array instead of a caller workspace, so its gradients
must equal attn_bwd's bit for bit.  Two calls in a row, the second on a
smaller problem (the array keeps the first call's D; the second must not read
it), plus a float32 call; torch's allocator must see no allocation during the
calls.
"""

import math

import pytest
import torch

import synth
from tests.gpu_util import upload

pytestmark = [pytest.mark.gpu]


def _api():
    import exact_io_aware_05_amd as E

    E.lib()
    return E


def _case(E, shape, dtype, causal, seed):
    print("[case] noalloc", shape, dtype, "causal" if causal else "full", "seed", seed, flush=True)
    inp = synth.qkvdo(seed, shape, dtype)
    q, k, v, do = (upload(inp[x + "_raw"], dtype) for x in ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(shape[3])
    o, lse = E.attn_fwd(q, k, v, causal=causal, scale=scale)
    ref = E.attn_bwd(q, k, v, o, do, lse, causal=causal, scale=scale)
    grads = tuple(torch.full_like(q, float("nan")) for _ in range(3))
    torch.cuda.synchronize()
    before = (torch.cuda.memory_allocated(), torch.cuda.max_memory_allocated())
    E.attn_bwd_noalloc(q, k, v, o, do, lse, grads, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert (torch.cuda.memory_allocated(), torch.cuda.max_memory_allocated()) == before
    for name, a, b in zip(("dQ", "dK", "dV"), ref, grads):
        view = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(a.view(view), b.view(view)), f"{name} differs from attn_bwd"


def test_noalloc_backward_equals_attn_bwd_on_consecutive_calls():
    E = _api()
    torch.cuda.reset_peak_memory_stats()
    _case(E, (2, 3, 1000, 128), "bf16", True, 71)
    _case(E, (1, 2, 300, 64), "bf16", False, 72)  # smaller: the array holds the first call's D
    _case(E, (1, 2, 200, 64), "fp32", True, 73)


def test_noalloc_backward_refuses_oversized_problems():
    E = _api()
    rows = E.NOALLOC_SCRATCH_BYTES // 4 // 64 + 1  # B * H * N just above the limit with B * H = 64
    q = torch.empty((64, 1, rows, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((64, 1, rows), dtype=torch.float32, device="cuda")
    with pytest.raises(E.AttnError) as ei:
        E.attn_bwd_noalloc(q, q, q, q, q, lse, (q, q, q), causal=True)
    assert ei.value.status == -9
