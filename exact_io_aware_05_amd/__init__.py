"""Fused exact attention for MI355X (gfx950): Python binding of ``libattn.so``.

The binding only marshals arguments: every step of the forward and backward
pass runs in the HIP kernels of the C library (``include/attn.h``).  PyTorch
tensors serve as device memory and the current HIP stream is passed through.
There is no fallback: if the library is missing, loading it raises.

Entry points carry the C names:

* :func:`attn_fwd` (q, k, v, causal, scale) -> (o, lse)
* :func:`attn_bwd` (q, k, v, o, do, lse, causal, scale) -> (dq, dk, dv)
* :func:`attn_bwd_dsum`, :func:`attn_bwd_dkdv`, :func:`attn_bwd_dq` -- the
  three phases of the backward pass, for use on separate streams or timing
* :func:`attn_fwd_blocksparse`, :func:`attn_bwd_blocksparse` -- the same
  with a block mask over 128 x 128 blocks of the score matrix
* :func:`attn_fwd_qk`, :func:`attn_bwd_qk` -- queries and keys of different
  lengths (bottom-right causal alignment), with split-K/V for the forward
* :func:`attn_fwd_dropout`, :func:`attn_bwd_dropout` -- the same with dropout
  on the probabilities (mask from a counter-based generator, not stored)
* :func:`attn_fwd_kpad`, :func:`attn_bwd_kpad` -- the same with a key padding
  mask (per-sequence key lengths)
* :func:`attn_fwd_window`, :func:`attn_bwd_window` -- causal attention over a
  sliding window of the last ``window`` keys
* :func:`attn_bwd_workspace_bytes`, :func:`attn_status_string`
* :func:`lib` -- the raw ``ctypes.CDLL``.

The cache-blocked multi-core CPU form of the same attention is a separate
library with its own binding, :mod:`exact_io_aware_05_amd.cpu`; nothing here
calls it.
"""

import ctypes
import math
import os

__all__ = [
    "attn_fwd",
    "attn_bwd",
    "attn_bwd_dsum",
    "attn_bwd_dkdv",
    "attn_bwd_dq",
    "attn_fwd_blocksparse",
    "attn_bwd_blocksparse",
    "SPARSE_BLOCK",
    "attn_fwd_qk",
    "attn_bwd_qk",
    "attn_fwd_dropout",
    "attn_bwd_dropout",
    "attn_fwd_kpad",
    "attn_bwd_kpad",
    "attn_fwd_window",
    "attn_bwd_window",
    "attn_bwd_workspace_bytes",
    "attn_status_string",
    "lib",
    "LIB_PATH",
    "ATTN_BF16",
    "ATTN_FP32",
    "AttnError",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

ATTN_BF16 = 0
ATTN_FP32 = 1
SPARSE_BLOCK = 128  # ATTN_SPARSE_BLOCK: rows per block of the block-sparse mask

_lib = None


class AttnError(RuntimeError):
    """A non-zero status returned by the C library."""

    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: status {status} ({attn_status_string(status)})")


def lib():
    """Load ``libattn.so`` (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m exact_io_aware_05_amd.build` "
            "(or __graft_entry__.build())"
        )
    # torch ships its own HIP runtime under the system's soname; with torch
    # loaded first the library binds to that one runtime, and device memory
    # and streams from torch are valid in it (a second runtime loaded beside
    # it would see no GPU once the first holds it).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, f32, vp]
    L.attn_fwd.restype = i32
    L.attn_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64, i32]
    L.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, f32, vp,
                           ctypes.c_size_t, vp]
    L.attn_bwd.restype = i32
    L.attn_bwd_dsum.argtypes = [vp, vp, vp, i64, i64, i64, i64, i32, vp]
    L.attn_bwd_dsum.restype = i32
    L.attn_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, f32, vp]
    L.attn_bwd_dkdv.restype = i32
    L.attn_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, f32, vp]
    L.attn_bwd_dq.restype = i32
    L.attn_fwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, f32, vp, i64, vp]
    L.attn_fwd_blocksparse.restype = i32
    L.attn_bwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, f32, vp,
                                       i64, vp, ctypes.c_size_t, vp]
    L.attn_bwd_blocksparse.restype = i32
    L.attn_fwd_qk_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i32, i32]
    L.attn_fwd_qk_workspace_bytes.restype = ctypes.c_size_t
    L.attn_fwd_qk.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i32, f32, i32, vp, ctypes.c_size_t,
                              vp]
    L.attn_fwd_qk.restype = i32
    L.attn_bwd_qk_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i32]
    L.attn_bwd_qk_workspace_bytes.restype = ctypes.c_size_t
    L.attn_bwd_qk.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i32, f32, vp,
                              ctypes.c_size_t, vp]
    L.attn_bwd_qk.restype = i32
    u64 = ctypes.c_uint64
    L.attn_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, f32, f32, u64, u64, vp]
    L.attn_fwd_dropout.restype = i32
    L.attn_bwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, f32, f32, u64,
                                   u64, vp, ctypes.c_size_t, vp]
    L.attn_bwd_dropout.restype = i32
    L.attn_bwd_dq_dsum.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, f32, vp]
    L.attn_bwd_dq_dsum.restype = i32
    L.attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, f32, vp]
    L.attn_bwd_noalloc.restype = i32
    L.attn_fwd_kpad.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, f32, vp, vp]
    L.attn_fwd_kpad.restype = i32
    L.attn_bwd_kpad.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, f32, vp, vp,
                                ctypes.c_size_t, vp]
    L.attn_bwd_kpad.restype = i32
    L.attn_fwd_window.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i64, f32, vp]
    L.attn_fwd_window.restype = i32
    L.attn_bwd_window.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i64, f32, vp,
                                  ctypes.c_size_t, vp]
    L.attn_bwd_window.restype = i32
    L.attn_status_string.argtypes = [i32]
    L.attn_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def attn_status_string(status):
    return lib().attn_status_string(int(status)).decode()


def attn_bwd_workspace_bytes(B, H, N, d, dtype):
    return int(lib().attn_bwd_workspace_bytes(B, H, N, d, dtype))


def _torch():
    import torch

    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_FP32
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _check(tensors, shape, dtype, device):
    for name, t in tensors:
        if t.shape != shape:
            raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
        if t.dtype != dtype:
            raise TypeError(f"{name}: dtype {t.dtype} != {dtype}")
        if t.device != device:
            raise ValueError(f"{name}: device {t.device} != {device}")
        if not t.is_contiguous():
            raise ValueError(f"{name}: must be contiguous [B, H, N, d]")


def _stream_ptr(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def attn_fwd(q, k, v, causal=False, scale=None, out=None, lse=None):
    """Fused attention forward on [B, H, N, d] GPU tensors; returns (o, lse).

    ``scale`` defaults to 1/sqrt(d).  ``o`` has the dtype of ``q``; ``lse`` is
    float32 [B, H, N].  Enqueued on the current stream.
    """
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    if not q.is_cuda:
        raise ValueError("tensors must be on a GPU")
    _check([("q", q), ("k", k), ("v", v)], q.shape, q.dtype, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check([("out", out)], q.shape, q.dtype, q.device)
    _check([("lse", lse)], (B, H, N), torch.float32, q.device)
    st = lib().attn_fwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
        B, H, N, d, _dtype_code(q), int(bool(causal)), float(scale), _stream_ptr(q.device),
    )
    if st != 0:
        raise AttnError(st, "attn_fwd")
    return out, lse


def attn_bwd(q, k, v, o, do, lse, causal=False, scale=None, workspace=None, grads=None):
    """Attention backward by recomputation; returns (dq, dk, dv).

    ``o`` and ``lse`` must come from :func:`attn_fwd` with the same
    ``causal`` and ``scale``.  ``workspace`` (a uint8 GPU tensor of at least
    :func:`attn_bwd_workspace_bytes` bytes) is allocated when not given.
    """
    torch = _torch()
    B, H, N, d = q.shape
    _check([("q", q), ("k", k), ("v", v), ("o", o), ("do", do)], q.shape, q.dtype, q.device)
    _check([("lse", lse)], (B, H, N), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = _dtype_code(q)
    need = attn_bwd_workspace_bytes(B, H, N, d, code)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = grads
    _check([("dq", dq), ("dk", dk), ("dv", dv)], q.shape, q.dtype, q.device)
    st = lib().attn_bwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, code, int(bool(causal)), float(scale),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream_ptr(q.device),
    )
    if st != 0:
        raise AttnError(st, "attn_bwd")
    return dq, dk, dv


NOALLOC_SCRATCH_BYTES = 16 << 20  # ATTN_NOALLOC_SCRATCH_BYTES in include/attn.h


def attn_bwd_noalloc(q, k, v, o, do, lse, grads, causal=False, scale=None):
    """:func:`attn_bwd` without any allocation: the caller passes the output
    tensors ``grads = (dq, dk, dv)``, and the library's scratch is a fixed
    device array (B * H * N <= NOALLOC_SCRATCH_BYTES / 4).  Calls that overlap
    on one GPU race on that array.  Returns ``grads``."""
    torch = _torch()
    B, H, N, d = q.shape
    _check([("q", q), ("k", k), ("v", v), ("o", o), ("do", do)], q.shape, q.dtype, q.device)
    _check([("lse", lse)], (B, H, N), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = grads
    _check([("dq", dq), ("dk", dk), ("dv", dv)], q.shape, q.dtype, q.device)
    st = lib().attn_bwd_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, _dtype_code(q), int(bool(causal)), float(scale),
        _stream_ptr(q.device),
    )
    if st != 0:
        raise AttnError(st, "attn_bwd_noalloc")
    return grads


def attn_bwd_dsum(o, do, dsum=None):
    """D_i = sum_k dO_ik O_ik into a float32 [B, H, N] tensor (returned)."""
    torch = _torch()
    B, H, N, d = o.shape
    _check([("o", o), ("do", do)], o.shape, o.dtype, o.device)
    if dsum is None:
        dsum = torch.empty((B, H, N), dtype=torch.float32, device=o.device)
    _check([("dsum", dsum)], (B, H, N), torch.float32, o.device)
    st = lib().attn_bwd_dsum(o.data_ptr(), do.data_ptr(), dsum.data_ptr(), B, H, N, d, _dtype_code(o),
                             _stream_ptr(o.device))
    if st != 0:
        raise AttnError(st, "attn_bwd_dsum")
    return dsum


def attn_bwd_dq_dsum(q, k, v, o, do, lse, causal=False, scale=None, dsum=None, dq=None):
    """dQ with D formed inside the dQ pass; returns (dq, dsum), dsum being
    float32 [B, H, N] (D_i = sum_k dO_ik O_ik) for :func:`attn_bwd_dkdv`."""
    torch = _torch()
    B, H, N, d = q.shape
    _check([("q", q), ("k", k), ("v", v), ("o", o), ("do", do)], q.shape, q.dtype, q.device)
    _check([("lse", lse)], (B, H, N), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if dsum is None:
        dsum = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if dq is None:
        dq = torch.empty_like(q)
    _check([("dsum", dsum)], (B, H, N), torch.float32, q.device)
    _check([("dq", dq)], q.shape, q.dtype, q.device)
    st = lib().attn_bwd_dq_dsum(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                lse.data_ptr(), dsum.data_ptr(), dq.data_ptr(), B, H, N, d, _dtype_code(q),
                                int(bool(causal)), float(scale), _stream_ptr(q.device))
    if st != 0:
        raise AttnError(st, "attn_bwd_dq_dsum")
    return dq, dsum


def attn_bwd_dkdv(q, k, v, do, lse, dsum, causal=False, scale=None, dk=None, dv=None):
    """dK and dV from the recomputed probabilities; returns (dk, dv)."""
    torch = _torch()
    B, H, N, d = q.shape
    _check([("q", q), ("k", k), ("v", v), ("do", do)], q.shape, q.dtype, q.device)
    _check([("lse", lse), ("dsum", dsum)], (B, H, N), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check([("dk", dk), ("dv", dv)], q.shape, q.dtype, q.device)
    st = lib().attn_bwd_dkdv(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(), dsum.data_ptr(), dk.data_ptr(),
        dv.data_ptr(), B, H, N, d, _dtype_code(q), int(bool(causal)), float(scale), _stream_ptr(q.device),
    )
    if st != 0:
        raise AttnError(st, "attn_bwd_dkdv")
    return dk, dv


def attn_bwd_dq(q, k, v, do, lse, dsum, causal=False, scale=None, dq=None):
    """dQ from the recomputed probabilities; returns dq."""
    torch = _torch()
    B, H, N, d = q.shape
    _check([("q", q), ("k", k), ("v", v), ("do", do)], q.shape, q.dtype, q.device)
    _check([("lse", lse), ("dsum", dsum)], (B, H, N), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    _check([("dq", dq)], q.shape, q.dtype, q.device)
    st = lib().attn_bwd_dq(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(), dsum.data_ptr(), dq.data_ptr(),
        B, H, N, d, _dtype_code(q), int(bool(causal)), float(scale), _stream_ptr(q.device),
    )
    if st != 0:
        raise AttnError(st, "attn_bwd_dq")
    return dq


def _block_mask(mask, B, H, N, device):
    """Validate a block mask tensor; returns (tensor, head stride in bytes).

    Accepted: uint8 or bool, contiguous, on ``device``, shaped [nb, nb] (one
    mask for every head), [B, H, nb, nb] or [B * H, nb, nb], with
    nb = ceil(N / 128).
    """
    torch = _torch()
    nb = (N + SPARSE_BLOCK - 1) // SPARSE_BLOCK
    if mask.dtype not in (torch.uint8, torch.bool):
        raise TypeError(f"block_mask: dtype {mask.dtype}; use torch.uint8 or torch.bool")
    if mask.device != device or not mask.is_contiguous():
        raise ValueError("block_mask must be a contiguous tensor on the inputs' device")
    if tuple(mask.shape) == (nb, nb):
        return mask, 0
    if tuple(mask.shape) in ((B, H, nb, nb), (B * H, nb, nb)):
        return mask, nb * nb
    raise ValueError(f"block_mask: shape {tuple(mask.shape)}; expected ({nb}, {nb}), "
                     f"({B}, {H}, {nb}, {nb}) or ({B * H}, {nb}, {nb})")


def attn_fwd_blocksparse(q, k, v, block_mask, causal=False, scale=None, out=None, lse=None):
    """Block-sparse forward: query i attends key j only where the 128 x 128
    block holding (i, j) is nonzero in ``block_mask`` (and j <= i if
    ``causal``).  Rows with no allowed key get O = 0, LSE = -inf.  bf16 only.
    Returns (o, lse)."""
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    _check([("q", q), ("k", k), ("v", v)], q.shape, q.dtype, q.device)
    mask, stride = _block_mask(block_mask, B, H, N, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check([("out", out)], q.shape, q.dtype, q.device)
    _check([("lse", lse)], (B, H, N), torch.float32, q.device)
    st = lib().attn_fwd_blocksparse(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d, _dtype_code(q),
        int(bool(causal)), float(scale), mask.data_ptr(), stride, _stream_ptr(q.device),
    )
    if st != 0:
        raise AttnError(st, "attn_fwd_blocksparse")
    return out, lse


def attn_bwd_blocksparse(q, k, v, o, do, lse, block_mask, causal=False, scale=None, workspace=None, grads=None):
    """Block-sparse backward (same mask and causal flag as the forward);
    returns (dq, dk, dv)."""
    torch = _torch()
    B, H, N, d = q.shape
    _check([("q", q), ("k", k), ("v", v), ("o", o), ("do", do)], q.shape, q.dtype, q.device)
    _check([("lse", lse)], (B, H, N), torch.float32, q.device)
    mask, stride = _block_mask(block_mask, B, H, N, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = _dtype_code(q)
    need = attn_bwd_workspace_bytes(B, H, N, d, code)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = grads
    _check([("dq", dq), ("dk", dk), ("dv", dv)], q.shape, q.dtype, q.device)
    st = lib().attn_bwd_blocksparse(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, code, int(bool(causal)), float(scale),
        mask.data_ptr(), stride, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream_ptr(q.device),
    )
    if st != 0:
        raise AttnError(st, "attn_bwd_blocksparse")
    return dq, dk, dv


def _qk_shapes(q, k, v):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, H, Nq, d] and k, v [B, H, Nk, d]")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    _check([("q", q)], (B, H, Nq, d), q.dtype, q.device)
    _check([("k", k), ("v", v)], (B, H, Nk, d), q.dtype, q.device)
    return B, H, Nq, Nk, d


def attn_fwd_qk(q, k, v, causal=False, scale=None, num_splits=1, out=None, lse=None, workspace=None):
    """Forward with Nq queries and Nk keys (bottom-right causal alignment:
    query i sees key j when j <= i + Nk - Nq).  ``num_splits``: 1 = one pass,
    2..64 = split-K/V into at most that many key chunks merged afterwards,
    0 = chosen from the shape.  bf16 only.  Returns (o, lse)."""
    torch = _torch()
    B, H, Nq, Nk, d = _qk_shapes(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = _dtype_code(q)
    need = int(lib().attn_fwd_qk_workspace_bytes(B, H, Nq, Nk, d, code, int(num_splits)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    _check([("out", out)], q.shape, q.dtype, q.device)
    _check([("lse", lse)], (B, H, Nq), torch.float32, q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().attn_fwd_qk(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, Nq, Nk, d, code,
        int(bool(causal)), float(scale), int(num_splits), ws_ptr, ws_bytes, _stream_ptr(q.device),
    )
    if st != 0:
        raise AttnError(st, "attn_fwd_qk")
    return out, lse


def attn_bwd_qk(q, k, v, o, do, lse, causal=False, scale=None, workspace=None, grads=None):
    """Backward for Nq queries and Nk keys (same causal and scale as the
    forward); returns (dq, dk, dv)."""
    torch = _torch()
    B, H, Nq, Nk, d = _qk_shapes(q, k, v)
    _check([("o", o), ("do", do)], q.shape, q.dtype, q.device)
    _check([("lse", lse)], (B, H, Nq), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = _dtype_code(q)
    need = int(lib().attn_bwd_qk_workspace_bytes(B, H, Nq, Nk, d, code))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = grads
    _check([("dq", dq)], q.shape, q.dtype, q.device)
    _check([("dk", dk), ("dv", dv)], k.shape, q.dtype, q.device)
    st = lib().attn_bwd_qk(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(), dq.data_ptr(),
        dk.data_ptr(), dv.data_ptr(), B, H, Nq, Nk, d, code, int(bool(causal)), float(scale),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream_ptr(q.device),
    )
    if st != 0:
        raise AttnError(st, "attn_bwd_qk")
    return dq, dk, dv


def attn_fwd_dropout(q, k, v, p_drop, seed, offset=0, causal=False, scale=None, out=None, lse=None):
    """Forward with dropout on the probabilities; returns (o, lse).  bf16 only.

    The keep mask is a function of (seed, offset, head, query, key); pass the
    same values to :func:`attn_bwd_dropout`."""
    torch = _torch()
    B, H, N, d = q.shape
    _check([("q", q), ("k", k), ("v", v)], q.shape, q.dtype, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    st = lib().attn_fwd_dropout(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d, _dtype_code(q),
        int(bool(causal)), float(scale), float(p_drop), int(seed), int(offset), _stream_ptr(q.device),
    )
    if st != 0:
        raise AttnError(st, "attn_fwd_dropout")
    return out, lse


def attn_bwd_dropout(q, k, v, o, do, lse, p_drop, seed, offset=0, causal=False, scale=None, workspace=None,
                     grads=None):
    """Backward of :func:`attn_fwd_dropout` (same p_drop, seed, offset, causal,
    scale); returns (dq, dk, dv)."""
    torch = _torch()
    B, H, N, d = q.shape
    _check([("q", q), ("k", k), ("v", v), ("o", o), ("do", do)], q.shape, q.dtype, q.device)
    _check([("lse", lse)], (B, H, N), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = _dtype_code(q)
    need = attn_bwd_workspace_bytes(B, H, N, d, code)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = grads
    st = lib().attn_bwd_dropout(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(), dq.data_ptr(),
        dk.data_ptr(), dv.data_ptr(), B, H, N, d, code, int(bool(causal)), float(scale), float(p_drop), int(seed),
        int(offset), workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream_ptr(q.device),
    )
    if st != 0:
        raise AttnError(st, "attn_bwd_dropout")
    return dq, dk, dv


def _key_len(key_len, B, device):
    torch = _torch()
    if not (torch.is_tensor(key_len) and key_len.dtype == torch.int32 and key_len.shape == (B,)
            and key_len.device == device and key_len.is_contiguous()):
        raise ValueError(f"key_len must be a contiguous int32 tensor of shape ({B},) on {device}")
    return key_len


def attn_fwd_kpad(q, k, v, key_len, causal=False, scale=None, out=None, lse=None):
    """Forward with a key padding mask: batch b attends only its keys
    j < key_len[b] (int32 [B] on the same GPU; clamped to [0, N] by the
    kernels).  Returns (o, lse); a row that sees no key gets o = 0 and
    lse = -inf."""
    torch = _torch()
    B, H, N, d = q.shape
    _check([("q", q), ("k", k), ("v", v)], q.shape, q.dtype, q.device)
    key_len = _key_len(key_len, B, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check([("out", out)], q.shape, q.dtype, q.device)
    _check([("lse", lse)], (B, H, N), torch.float32, q.device)
    st = lib().attn_fwd_kpad(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d, _dtype_code(q),
        int(bool(causal)), float(scale), key_len.data_ptr(), _stream_ptr(q.device),
    )
    if st != 0:
        raise AttnError(st, "attn_fwd_kpad")
    return out, lse


def attn_bwd_kpad(q, k, v, o, do, lse, key_len, causal=False, scale=None, workspace=None, grads=None):
    """Backward of :func:`attn_fwd_kpad` (same key_len, causal, scale);
    returns (dq, dk, dv), with dk = dv = 0 for the padded keys."""
    torch = _torch()
    B, H, N, d = q.shape
    _check([("q", q), ("k", k), ("v", v), ("o", o), ("do", do)], q.shape, q.dtype, q.device)
    _check([("lse", lse)], (B, H, N), torch.float32, q.device)
    key_len = _key_len(key_len, B, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = _dtype_code(q)
    need = attn_bwd_workspace_bytes(B, H, N, d, code)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = grads
    _check([("dq", dq), ("dk", dk), ("dv", dv)], q.shape, q.dtype, q.device)
    st = lib().attn_bwd_kpad(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(), dq.data_ptr(),
        dk.data_ptr(), dv.data_ptr(), B, H, N, d, code, int(bool(causal)), float(scale), key_len.data_ptr(),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream_ptr(q.device),
    )
    if st != 0:
        raise AttnError(st, "attn_bwd_kpad")
    return dq, dk, dv


def attn_fwd_window(q, k, v, window, scale=None, out=None, lse=None):
    """Causal attention over a sliding window: query i attends keys
    i - window < j <= i.  Returns (o, lse)."""
    torch = _torch()
    B, H, N, d = q.shape
    _check([("q", q), ("k", k), ("v", v)], q.shape, q.dtype, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check([("out", out)], q.shape, q.dtype, q.device)
    _check([("lse", lse)], (B, H, N), torch.float32, q.device)
    st = lib().attn_fwd_window(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d, _dtype_code(q),
        int(window), float(scale), _stream_ptr(q.device),
    )
    if st != 0:
        raise AttnError(st, "attn_fwd_window")
    return out, lse


def attn_bwd_window(q, k, v, o, do, lse, window, scale=None, workspace=None, grads=None):
    """Backward of :func:`attn_fwd_window` (same window and scale); returns
    (dq, dk, dv)."""
    torch = _torch()
    B, H, N, d = q.shape
    _check([("q", q), ("k", k), ("v", v), ("o", o), ("do", do)], q.shape, q.dtype, q.device)
    _check([("lse", lse)], (B, H, N), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = _dtype_code(q)
    need = attn_bwd_workspace_bytes(B, H, N, d, code)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = grads
    _check([("dq", dq), ("dk", dk), ("dv", dv)], q.shape, q.dtype, q.device)
    st = lib().attn_bwd_window(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(), dq.data_ptr(),
        dk.data_ptr(), dv.data_ptr(), B, H, N, d, code, int(window), float(scale), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream_ptr(q.device),
    )
    if st != 0:
        raise AttnError(st, "attn_bwd_window")
    return dq, dk, dv
