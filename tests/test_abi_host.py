"""Host-only checks of the C ABI: the library loads, exports every declared
symbol, and rejects invalid arguments before touching a device."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def _lib():
    import exact_io_aware_05_amd as E

    if not os.path.exists(E.LIB_PATH):
        pytest.skip("libattn.so not built")
    return E, E.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == [
        "attn_bwd",
        "attn_bwd_blocksparse",
        "attn_bwd_dkdv",
        "attn_bwd_dq",
        "attn_bwd_dq_dsum",
        "attn_bwd_dropout",
        "attn_bwd_dsum",
        "attn_bwd_kpad",
        "attn_bwd_noalloc",
        "attn_bwd_qk",
        "attn_bwd_qk_workspace_bytes",
        "attn_bwd_window",
        "attn_bwd_workspace_bytes",
        "attn_fwd",
        "attn_fwd_blocksparse",
        "attn_fwd_dropout",
        "attn_fwd_kpad",
        "attn_fwd_qk",
        "attn_fwd_qk_workspace_bytes",
        "attn_fwd_window",
        "attn_status_string",
    ]


def test_library_exports_every_declared_symbol():
    _, L = _lib()
    raw = ctypes.CDLL(L._name)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_status_strings():
    E, _ = _lib()
    for st in range(-9, 1):
        s = E.attn_status_string(st)
        assert isinstance(s, str) and s and s != "unknown status"
    assert E.attn_status_string(-99) == "unknown status"


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _fwd(L, ptrs=(FAKE,) * 5, B=1, H=1, N=16, d=64, dtype=0, causal=0, scale=0.125):
    return L.attn_fwd(*ptrs, B, H, N, d, dtype, causal, scale, None)


def test_forward_argument_validation():
    E, L = _lib()
    for i in range(5):
        ptrs = [FAKE] * 5
        ptrs[i] = None
        assert _fwd(L, ptrs=ptrs) == -1
    assert _fwd(L, d=32) == -3
    assert _fwd(L, d=96) == -3
    assert _fwd(L, d=256) == -3
    assert _fwd(L, dtype=2) == -3
    assert _fwd(L, B=0) == -2
    assert _fwd(L, H=-1) == -2
    assert _fwd(L, N=0) == -2
    assert _fwd(L, N=2**31) == -2
    assert _fwd(L, B=2**16, H=2**16, N=2) == -2
    assert _fwd(L, N=2**24, d=128) == -2
    assert _fwd(L, N=2**23 + 1, d=128) == -2
    assert _fwd(L, scale=float("nan")) == -4
    assert _fwd(L, scale=float("inf")) == -4


def _bwd(L, ptrs=(FAKE,) * 9, B=1, H=1, N=16, d=64, dtype=0, causal=0, scale=0.125, ws=FAKE * 256, wsb=None):
    if wsb is None:
        wsb = L.attn_bwd_workspace_bytes(B, H, N, d, dtype)
    return L.attn_bwd(*ptrs, B, H, N, d, dtype, causal, scale, ws, wsb, None)


def test_backward_argument_validation():
    E, L = _lib()
    for i in range(9):
        ptrs = [FAKE] * 9
        ptrs[i] = None
        assert _bwd(L, ptrs=ptrs) == -1
    assert _bwd(L, d=80) == -3
    assert _bwd(L, dtype=7) == -3
    assert _bwd(L, N=0) == -2
    assert _bwd(L, scale=float("-inf")) == -4
    assert _bwd(L, ws=None) == -5
    assert _bwd(L, wsb=L.attn_bwd_workspace_bytes(1, 1, 16, 64, 0) - 1) == -5
    assert _bwd(L, ws=FAKE * 256 + 4) == -5  # misaligned


def test_backward_phase_validation():
    E, L = _lib()
    assert L.attn_bwd_dsum(None, FAKE, FAKE, 1, 1, 16, 64, 0, None) == -1
    assert L.attn_bwd_dsum(FAKE, FAKE, FAKE, 1, 1, 16, 48, 0, None) == -3
    assert L.attn_bwd_dsum(FAKE, FAKE, FAKE, 1, 0, 16, 64, 0, None) == -2
    for i in range(8):
        ptrs = [FAKE] * 8
        ptrs[i] = None
        assert L.attn_bwd_dkdv(*ptrs, 1, 1, 16, 64, 0, 0, 0.1, None) == -1
    assert L.attn_bwd_dkdv(*([FAKE] * 8), 1, 1, 16, 64, 3, 0, 0.1, None) == -3
    assert L.attn_bwd_dkdv(*([FAKE] * 8), 1, 1, 16, 64, 0, 0, float("nan"), None) == -4
    for i in range(7):
        ptrs = [FAKE] * 7
        ptrs[i] = None
        assert L.attn_bwd_dq(*ptrs, 1, 1, 16, 64, 0, 1, 0.1, None) == -1
    assert L.attn_bwd_dq(*([FAKE] * 7), 1, 1, 0, 64, 0, 1, 0.1, None) == -2
    assert L.attn_bwd_dq(*([FAKE] * 7), 1, 1, 16, 64, 0, 1, float("inf"), None) == -4


def test_dq_dsum_validation():
    _, L = _lib()

    def call(ptrs=(FAKE,) * 8, N=16, d=64, dtype=0, scale=0.1):
        return L.attn_bwd_dq_dsum(*ptrs, 1, 2, N, d, dtype, 1, scale, None)

    for i in range(8):
        ptrs = [FAKE] * 8
        ptrs[i] = None
        assert call(ptrs=ptrs) == -1
    ptrs = [FAKE] * 8
    ptrs[6] = FAKE + 2  # dsum: 4-byte alignment
    assert call(ptrs=ptrs) == -8
    ptrs = [FAKE] * 8
    ptrs[3] = FAKE + 2  # o
    assert call(ptrs=ptrs) == -8
    assert call(d=32) == -3 and call(N=0) == -2 and call(scale=float("inf")) == -4


def test_noalloc_backward_validation():
    """attn_bwd_noalloc validates like attn_bwd, and refuses problems whose
    D (4 * B * H * N bytes) exceeds its fixed scratch, before any HIP call."""
    E, L = _lib()

    def call(ptrs=(FAKE,) * 9, B=1, H=1, N=16, d=64, dtype=0, scale=0.1):
        return L.attn_bwd_noalloc(*ptrs, B, H, N, d, dtype, 1, scale, None)

    for i in range(9):
        ptrs = [FAKE] * 9
        ptrs[i] = None
        assert call(ptrs=ptrs) == -1
    ptrs = [FAKE] * 9
    ptrs[0] = FAKE + 2
    assert call(ptrs=ptrs) == -8
    assert call(d=96) == -3 and call(N=0) == -2 and call(scale=float("nan")) == -4
    m = re.search(r"#define ATTN_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == E.NOALLOC_SCRATCH_BYTES
    limit = E.NOALLOC_SCRATCH_BYTES // 4  # rows of D
    assert call(B=1, H=1, N=limit + 1) == -9
    assert call(B=64, H=1, N=limit // 64 + 1) == -9
    assert E.attn_status_string(-9) != "unknown status"


def test_misaligned_pointers_are_refused():
    """Tensor pointers must be 16-byte aligned and LSE / D pointers 4-byte
    aligned (the kernels use 16-byte vector and buffer->LDS accesses): a
    pointer off by one bf16 element, as a contiguous view at an odd storage
    offset would give, is refused with ATTN_E_ALIGN (-8) before any HIP call."""
    _, L = _lib()
    odd = FAKE + 2  # a valid bf16 address, not 16-byte aligned
    for i in range(4):  # q, k, v, o
        ptrs = [FAKE] * 5
        ptrs[i] = odd
        assert _fwd(L, ptrs=ptrs) == -8
    assert _fwd(L, ptrs=[FAKE] * 4 + [FAKE + 2]) == -8  # LSE at 2 bytes
    for i in range(9):
        ptrs = [FAKE] * 9
        ptrs[i] = FAKE + (2 if i != 5 else 1)  # index 5 is LSE
        assert _bwd(L, ptrs=ptrs) == -8, i
    assert L.attn_bwd_dsum(FAKE, FAKE, FAKE + 2, 1, 1, 16, 64, 0, None) == -8
    assert L.attn_bwd_dsum(odd, FAKE, FAKE, 1, 1, 16, 64, 0, None) == -8
    dk = [FAKE] * 8
    dk[6] = odd
    assert L.attn_bwd_dkdv(*dk, 1, 1, 16, 64, 0, 0, 0.1, None) == -8
    dq = [FAKE] * 7
    dq[5] = FAKE + 1  # D
    assert L.attn_bwd_dq(*dq, 1, 1, 16, 64, 0, 1, 0.1, None) == -8
    bs = [FAKE] * 5
    bs[2] = odd
    assert L.attn_fwd_blocksparse(*bs, 1, 1, 300, 64, 0, 0, 0.1, FAKE + 1, 0, None) == -8
    qk = [FAKE] * 5
    qk[3] = odd
    assert L.attn_fwd_qk(*qk, 1, 1, 5, 300, 64, 0, 1, 0.1, 1, None, 0, None) == -8
    dr = [FAKE] * 5
    dr[0] = odd
    assert L.attn_fwd_dropout(*dr, 1, 1, 16, 64, 0, 0, 0.1, 0.1, 1, 0, None) == -8


def test_blocksparse_argument_validation():
    E, L = _lib()

    def fwd(ptrs=(FAKE,) * 5, B=2, H=3, N=300, d=64, dtype=0, mask=FAKE, stride=0, scale=0.1):
        return L.attn_fwd_blocksparse(*ptrs, B, H, N, d, dtype, 0, scale, mask, stride, None)

    def bwd(ptrs=(FAKE,) * 9, B=2, H=3, N=300, d=64, dtype=0, mask=FAKE, stride=0, ws=FAKE * 256, wsb=None):
        if wsb is None:
            wsb = L.attn_bwd_workspace_bytes(B, H, N, d, 0)
        return L.attn_bwd_blocksparse(*ptrs, B, H, N, d, dtype, 1, 0.1, mask, stride, ws, wsb, None)

    nb = 3  # ceil(300 / 128)
    for i in range(5):
        ptrs = [FAKE] * 5
        ptrs[i] = None
        assert fwd(ptrs=ptrs) == -1
    for i in range(9):
        ptrs = [FAKE] * 9
        ptrs[i] = None
        assert bwd(ptrs=ptrs) == -1
    assert fwd(mask=None) == -1 and bwd(mask=None) == -1
    assert fwd(dtype=1) == -3 and bwd(dtype=1) == -3  # bf16 only
    assert fwd(d=96) == -3 and fwd(N=0) == -2
    assert fwd(N=131073) == -2 and bwd(N=131073) == -2  # beyond ATTN_SPARSE_MAX_N
    assert fwd(stride=-1) == -2 and bwd(stride=nb * nb - 1) == -2
    assert fwd(stride=2**62) == -2  # last head's mask not addressable
    assert fwd(scale=float("nan")) == -4
    assert bwd(ws=None) == -5 and bwd(ws=FAKE * 256 + 8) == -5
    assert E.SPARSE_BLOCK == 128


def test_unequal_lengths_validation_and_workspace():
    E, L = _lib()

    def fwd(ptrs=(FAKE,) * 5, Nq=5, Nk=300, dtype=0, splits=1, ws=None, wsb=0, scale=0.1):
        return L.attn_fwd_qk(*ptrs, 2, 3, Nq, Nk, 64, dtype, 1, scale, splits, ws, wsb, None)

    def bwd(ptrs=(FAKE,) * 9, Nq=5, Nk=300, dtype=0, ws=FAKE * 256, wsb=None):
        if wsb is None:
            wsb = L.attn_bwd_qk_workspace_bytes(2, 3, Nq, Nk, 64, 0)
        return L.attn_bwd_qk(*ptrs, 2, 3, Nq, Nk, 64, dtype, 1, 0.1, ws, wsb, None)

    for i in range(5):
        ptrs = [FAKE] * 5
        ptrs[i] = None
        assert fwd(ptrs=ptrs) == -1
    for i in range(9):
        ptrs = [FAKE] * 9
        ptrs[i] = None
        assert bwd(ptrs=ptrs) == -1
    assert fwd(dtype=1) == -3 and bwd(dtype=1) == -3
    assert fwd(Nq=0) == -2 and fwd(Nk=0) == -2 and bwd(Nk=2**31) == -2
    assert fwd(splits=-1) == -2 and fwd(splits=65) == -2
    assert fwd(scale=float("nan")) == -4
    # A split needs a workspace: sized by the query, refused when absent or short.
    need = L.attn_fwd_qk_workspace_bytes(2, 3, 5, 300, 64, 0, 4)
    rows = 2 * 3 * 5 * 4  # 300 keys = 5 tiles; at most 4 chunks of 2 tiles -> 3 chunks
    assert need > 0 and need % 256 == 0
    assert need == L.attn_fwd_qk_workspace_bytes(2, 3, 5, 300, 64, 0, 3)
    assert need <= ((rows * 64 * 4 + 255) // 256 + (rows * 4 + 255) // 256) * 256
    assert fwd(splits=4) == -5 and fwd(splits=4, ws=FAKE * 256, wsb=need - 1) == -5
    assert fwd(splits=4, ws=FAKE * 256 + 16, wsb=need) == -5
    assert L.attn_fwd_qk_workspace_bytes(2, 3, 5, 300, 64, 0, 1) == 0
    assert L.attn_fwd_qk_workspace_bytes(2, 3, 5, 64, 64, 0, 8) == 0  # one key tile: nothing to split
    assert L.attn_fwd_qk_workspace_bytes(2, 3, 5, 300, 64, 1, 4) == 0  # fp32: invalid
    assert bwd(ws=None) == -5 and bwd(wsb=L.attn_bwd_qk_workspace_bytes(2, 3, 5, 300, 64, 0) - 1) == -5
    assert L.attn_bwd_qk_workspace_bytes(2, 3, 5, 300, 64, 0) == ((2 * 3 * 5 * 4 + 255) // 256) * 256


def test_unequal_lengths_backward_workspace_holds_the_dq_split():
    # With few (head, query block) workgroups (256 query rows each at d = 128,
    # 128 at d = 64) the dQ pass is split over chunks of whole 64-key tiles,
    # about 256 workgroups in all and at least 4 tiles a chunk; the workspace
    # adds one fp32 [B, H, Nq, d] partial per chunk after D.
    _, L = _lib()

    def dbytes(B, H, nq):
        return -(-(B * H * nq * 4) // 256) * 256

    # Chunked prefill: 64 workgroups, 128 tiles -> 4 chunks of 32 tiles.
    assert L.attn_bwd_qk_workspace_bytes(1, 16, 1024, 8192, 128, 0) == dbytes(1, 16, 1024) + 4 * 16 * 1024 * 128 * 4
    # Decoding: 8 workgroups, 79 tiles -> at most 19 chunks of 5 tiles -> 16.
    assert L.attn_bwd_qk_workspace_bytes(2, 4, 1, 5000, 128, 0) == dbytes(2, 4, 1) + 16 * 8 * 1 * 128 * 4
    # d = 64: 4 workgroups, 64 tiles -> 16 chunks of 4 tiles.
    assert L.attn_bwd_qk_workspace_bytes(2, 2, 64, 4096, 64, 0) == dbytes(2, 2, 64) + 16 * 4 * 64 * 64 * 4
    # Enough workgroups already (1024; 256 too): no split, D only.
    assert L.attn_bwd_qk_workspace_bytes(4, 16, 4096, 8192, 128, 0) == dbytes(4, 16, 4096)
    assert L.attn_bwd_qk_workspace_bytes(1, 16, 4096, 8192, 128, 0) == dbytes(1, 16, 4096)
    # Fewer than 8 key tiles: no chunk of 4 tiles to split off.
    assert L.attn_bwd_qk_workspace_bytes(1, 1, 1, 7 * 64, 128, 0) == dbytes(1, 1, 1)


def test_decode_forward_split_plan():
    # One to four query rows over at least as many keys take the decode
    # kernel, whose automatic split aims at about 1024 workgroups with chunks
    # of at least one pass of its waves (128 keys at d = 128, 256 at d = 64);
    # more rows keep the matrix-core plan (about 512 workgroups of 128 rows,
    # at least 4 tiles a chunk).  Workspace: fp32 O and LSE per row and chunk.
    _, L = _lib()

    def wsb(B, H, nq, chunks, d):
        rows = B * H * nq * chunks
        return -(-(rows * d * 4) // 256) * 256 + -(-(rows * 4) // 256) * 256

    # 8 heads, 79 tiles: at most 128 chunks by workgroups, 39 of 2 tiles -> 27 of 3.
    assert L.attn_fwd_qk_workspace_bytes(2, 4, 1, 5000, 128, 0, 0) == wsb(2, 4, 1, 27, 128)
    assert L.attn_fwd_qk_workspace_bytes(2, 4, 4, 5000, 128, 0, 0) == wsb(2, 4, 4, 27, 128)
    # Five rows: the matrix-core plan, 19 chunks of 4 tiles -> 16 of 5.
    assert L.attn_fwd_qk_workspace_bytes(2, 4, 5, 5000, 128, 0, 0) == wsb(2, 4, 5, 16, 128)
    # d = 64: chunks of at least 4 tiles; 32 heads, 64 tiles -> 16 chunks.
    assert L.attn_fwd_qk_workspace_bytes(1, 32, 1, 4096, 64, 0, 0) == wsb(1, 32, 1, 16, 64)
    # 32 heads at d = 128 over 4096 keys: 32 chunks of 2 tiles.
    assert L.attn_fwd_qk_workspace_bytes(1, 32, 1, 4096, 128, 0, 0) == wsb(1, 32, 1, 32, 128)
    # Enough heads for the chip: no split.
    assert L.attn_fwd_qk_workspace_bytes(16, 64, 1, 4096, 128, 0, 0) == 0
    # Chunked prefill, 1024 queries after 7168 keys, 16 heads: 128 workgroups
    # of 128 rows -> 4 chunks of 32 tiles (about 512 workgroups).
    assert L.attn_fwd_qk_workspace_bytes(1, 16, 1024, 8192, 128, 0, 0) == wsb(1, 16, 1024, 4, 128)
    # 512 workgroups already: no split.
    assert L.attn_fwd_qk_workspace_bytes(4, 16, 1024, 8192, 128, 0, 0) == 0
    # Explicit counts are honoured as for more rows.
    assert L.attn_fwd_qk_workspace_bytes(2, 4, 1, 5000, 128, 0, 8) == wsb(2, 4, 1, 8, 128)


def test_workspace_size():
    E, L = _lib()
    assert E.attn_bwd_workspace_bytes(2, 3, 100, 64, 0) >= 2 * 3 * 100 * 4
    assert E.attn_bwd_workspace_bytes(2, 3, 100, 64, 0) % 256 == 0
    assert E.attn_bwd_workspace_bytes(0, 3, 100, 64, 0) == 0
    assert E.attn_bwd_workspace_bytes(1, 1, 100, 48, 0) == 0


def test_product_path_does_not_use_the_oracle():
    """The package and its sources never reference the oracle."""
    pkg = os.path.join(ROOT, "exact_io_aware_05_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text, os.path.join(dirpath, f)


def test_dropout_arguments_are_validated_before_any_launch():
    E, L = _lib()
    f = [FAKE] * 5
    assert L.attn_fwd_dropout(None, *f[1:], 1, 1, 16, 64, 0, 0, 0.1, 0.1, 1, 0, None) == -1
    assert L.attn_fwd_dropout(*f, 1, 1, 16, 64, 1, 0, 0.1, 0.1, 1, 0, None) == -3  # fp32: unsupported
    assert L.attn_fwd_dropout(*f, 1, 1, 16, 48, 0, 0, 0.1, 0.1, 1, 0, None) == -3
    assert L.attn_fwd_dropout(*f, 1, 1, 16, 64, 0, 0, float("inf"), 0.1, 1, 0, None) == -4
    for p in (-0.1, 1.0, 1.5, float("nan")):
        assert L.attn_fwd_dropout(*f, 1, 1, 16, 64, 0, 0, 0.1, p, 1, 0, None) == -7
    g = [FAKE] * 9
    assert L.attn_bwd_dropout(*g, 1, 1, 16, 64, 0, 0, 0.1, 1.0, 1, 0, FAKE, 1 << 20, None) == -7
    assert L.attn_bwd_dropout(*g, 1, 1, 16, 64, 0, 0, 0.1, 0.2, 1, 0, None, 1 << 20, None) == -5
    assert L.attn_bwd_dropout(*g, 1, 1, 16, 64, 0, 0, 0.1, 0.2, 1, 0, FAKE, 16, None) == -5
    assert E.attn_status_string(-7).startswith("dropout probability")


def test_key_padding_arguments_are_validated_before_any_launch():
    E, L = _lib()
    f = [FAKE] * 5
    # NULL key lengths, misaligned key lengths, bad shape, bad scale.
    assert L.attn_fwd_kpad(*f, 1, 1, 16, 64, 0, 0, 0.1, None, None) == -1
    assert L.attn_fwd_kpad(*f, 1, 1, 16, 64, 0, 0, 0.1, FAKE + 2, None) == -8
    assert L.attn_fwd_kpad(*f, 1, 1, 16, 48, 0, 0, 0.1, FAKE, None) == -3
    assert L.attn_fwd_kpad(*f, 1, 1, 16, 64, 0, 0, float("nan"), FAKE, None) == -4
    g = [FAKE] * 9
    assert L.attn_bwd_kpad(*g, 1, 1, 16, 64, 0, 0, 0.1, None, FAKE, 1 << 20, None) == -1
    assert L.attn_bwd_kpad(*g, 1, 1, 16, 64, 0, 0, 0.1, FAKE + 2, FAKE, 1 << 20, None) == -8
    assert L.attn_bwd_kpad(*g, 1, 1, 16, 64, 0, 0, 0.1, FAKE, None, 1 << 20, None) == -5
    assert L.attn_bwd_kpad(*g, 1, 1, 16, 64, 0, 0, 0.1, FAKE, FAKE, 16, None) == -5


def test_window_arguments_are_validated_before_any_launch():
    E, L = _lib()
    f = [FAKE] * 5
    assert L.attn_fwd_window(None, *f[1:], 1, 1, 16, 64, 0, 4, 0.1, None) == -1
    assert L.attn_fwd_window(*f, 1, 1, 16, 64, 0, 0, 0.1, None) == -2
    assert L.attn_fwd_window(*f, 1, 1, 16, 64, 0, -3, 0.1, None) == -2
    assert L.attn_fwd_window(*f, 1, 1, 16, 96, 0, 4, 0.1, None) == -3
    assert L.attn_fwd_window(*f, 1, 1, 16, 64, 0, 4, float("inf"), None) == -4
    g = [FAKE] * 9
    assert L.attn_bwd_window(*g, 1, 1, 16, 64, 0, 0, 0.1, FAKE, 1 << 20, None) == -2
    assert L.attn_bwd_window(*g, 1, 1, 16, 64, 0, 4, 0.1, None, 1 << 20, None) == -5
    assert L.attn_bwd_window(*g, 1, 1, 16, 64, 0, 4, 0.1, FAKE, 16, None) == -5
    assert "window" in E.attn_status_string(-2)
