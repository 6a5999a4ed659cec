"""Seeded synthetic inputs for attention, shared by the tests, the bench and smoke.

This module holds no attention arithmetic.  It draws standard-normal float32
values with numpy's PCG64 generator and encodes them as bfloat16 bit patterns
(round to nearest, ties to even), so that the float64 oracle and the GPU
kernels receive bit-identical inputs.

Recipe (one call of :func:`qkvdo`): ``rng = np.random.Generator(np.random.PCG64(seed))``,
then ``rng.standard_normal(shape, dtype=np.float32)`` four times, in the order
Q, K, V, dO, each of shape ``[B, H, N, d]``.  For bf16 workloads each float32
value is rounded to bf16; the float64 arrays handed to the oracle are the exact
values of those bf16 numbers.
"""

import numpy as np

__all__ = [
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "qkvdo",
    "Workload",
    "WORKLOADS",
    "sample_pairs",
    "peaked_inputs",
    "ramp_inputs",
]


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    rounding = ((u >> 16) & 1) + 0x7FFF
    r = ((u + rounding) >> 16).astype(np.uint16)
    r = np.where(nan, np.uint16(0x7FC0), r)
    return r


def bf16_bits_to_f32(b):
    """Exact float32 values of bfloat16 bit patterns."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def qkvdo(seed, shape, dtype="bf16", with_do=True):
    """Draw (Q, K, V, dO) of ``shape`` = [B, H, N, d].

    Returns a dict with, per tensor name, ``"<name>"`` (float64 values for the
    oracle) and ``"<name>_raw"`` (the array to upload: uint16 bf16 bits for
    ``dtype == "bf16"``, float32 for ``dtype == "fp32"``).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    names = ["q", "k", "v", "do"] if with_do else ["q", "k", "v"]
    out = {}
    for name in names:
        x = rng.standard_normal(tuple(shape), dtype=np.float32)
        if dtype == "bf16":
            bits = f32_to_bf16_bits(x)
            out[name + "_raw"] = bits
            out[name] = bf16_bits_to_f32(bits).astype(np.float64)
        elif dtype == "fp32":
            out[name + "_raw"] = x
            out[name] = x.astype(np.float64)
        else:
            raise ValueError("dtype must be 'bf16' or 'fp32'")
    return out


def block_mask(seed, nb, density, heads=None):
    """Seeded uint8 block mask [nb, nb] (or [heads, nb, nb]) with each block
    kept with probability ``density`` (numpy PCG64, uniform draws)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (nb, nb) if heads is None else (heads, nb, nb)
    return (rng.random(shape) < density).astype(np.uint8)


class Workload:
    """One named attention workload: shape, dtype, mask and seed."""

    def __init__(self, name, b, h, n, d, dtype, causal, seed, passes):
        self.name = name
        self.b, self.h, self.n, self.d = b, h, n, d
        self.dtype = dtype
        self.causal = causal
        self.seed = seed
        self.passes = passes  # subset of ("fwd", "bwd")

    @property
    def shape(self):
        return (self.b, self.h, self.n, self.d)

    def __repr__(self):
        return (
            f"Workload({self.name}: B={self.b} H={self.h} N={self.n} d={self.d} "
            f"{self.dtype} causal={self.causal} seed={self.seed} {self.passes})"
        )


# The five workloads the method is measured and checked on.  Seeds are fixed
# so every consumer draws the same inputs.
WORKLOADS = {
    "fp32_n256_d64": Workload("fp32_n256_d64", 1, 1, 256, 64, "fp32", False, 1, ("fwd",)),
    "gpt2s_n1024_d64_causal": Workload("gpt2s_n1024_d64_causal", 8, 12, 1024, 64, "bf16", True, 2, ("fwd",)),
    "n4096_d128": Workload("n4096_d128", 4, 16, 4096, 128, "bf16", False, 3, ("fwd",)),
    "n4096_d128_causal": Workload("n4096_d128_causal", 4, 16, 4096, 128, "bf16", True, 3, ("fwd",)),
    "bwd_n2048_d64_causal": Workload("bwd_n2048_d64_causal", 8, 16, 2048, 64, "bf16", True, 4, ("fwd", "bwd")),
    "long_n65536_d64_causal": Workload("long_n65536_d64_causal", 1, 8, 65536, 64, "bf16", True, 5, ("fwd", "bwd")),
}


def sample_pairs(seed, heads, n, count):
    """``count`` distinct (head, row) pairs drawn uniformly from heads x n, sorted."""
    rng = np.random.Generator(np.random.PCG64(seed))
    flat = rng.choice(heads * n, size=count, replace=False)
    flat.sort()
    return np.stack([flat // n, flat % n], axis=1)


def ramp_inputs(seed, shape, slope=1.0, height=8.0):
    """(Q, K, V) of ``shape`` whose scores rise along every row: feature 0 of
    every query is ``height`` and of key j is ``slope * j`` (rounded to bf16,
    so equal within runs of a few keys at large j); the other features and V
    are standard normal.  Returned as in :func:`qkvdo`."""
    b, h, n, d = shape
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    q[..., 0] = height
    k[..., 0] = slope * np.arange(n, dtype=np.float32)
    out = {}
    for name, x in (("q", q), ("k", k), ("v", v)):
        bits = f32_to_bf16_bits(x)
        out[name + "_raw"] = bits
        out[name] = bf16_bits_to_f32(bits).astype(np.float64)
    return out


def peaked_inputs(seed, shape, product, q_over_k=9.0, do_scale=1.0):
    """(Q, K, V, dO) of ``shape`` = [B, H, N, d] whose score rows rise toward a
    chosen key.

    Features 0 and 1 of key j are ``rk * (cos t_j, sin t_j)`` with
    ``t_j = 2 pi j / N``; those of query i are ``rq * (cos t_p, sin t_p)`` for
    a key p drawn uniformly per query (every eighth query takes one of the
    last 64 keys instead), with ``rq * rk = product`` and
    ``rq / rk = q_over_k``.  Their contribution to the dot product is
    ``product * cos(t_j - t_p)``, so along a row it climbs toward key p and
    falls after it.  The other features of Q and K, and V, are standard
    normal; dO is standard normal times ``do_scale``.  Values are rounded to
    bf16 and returned as in :func:`qkvdo` (``"<name>"`` float64 values,
    ``"<name>_raw"`` uint16 bits).
    """
    b, h, n, d = shape
    rq = float(np.sqrt(product * q_over_k))
    rk = float(np.sqrt(product / q_over_k))
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    do = rng.standard_normal(shape, dtype=np.float32) * np.float32(do_scale)
    peak = rng.integers(0, n, size=(b, h, n))
    rows = np.arange(n)
    late = rows % 8 == 0
    peak[..., late] = np.maximum(n - 1 - rows[late] % 64, 0)
    tk = 2.0 * np.pi * np.arange(n) / n
    tq = 2.0 * np.pi * peak / n
    k[..., 0] = rk * np.cos(tk)
    k[..., 1] = rk * np.sin(tk)
    q[..., 0] = rq * np.cos(tq)
    q[..., 1] = rq * np.sin(tq)
    out = {}
    for name, x in (("q", q), ("k", k), ("v", v), ("do", do)):
        bits = f32_to_bf16_bits(x)
        out[name + "_raw"] = bits
        out[name] = bf16_bits_to_f32(bits).astype(np.float64)
    return out
