"""GPU parity of attention with unequal query and key lengths (bottom-right
causal alignment) and of the split-K/V forward, through the C ABI, against
the float64 oracle of oracle/varlen.py."""

import math

import numpy as np
import pytest
import torch

import synth
from oracle import varlen as VL
from tests.gpu_util import assert_close, download, upload

pytestmark = [pytest.mark.gpu]


def _api():
    import exact_io_aware_05_amd as E

    E.lib()
    return E


def _announce(*a):
    print("[case]", *a, flush=True)


def _inputs(seed, B, H, nq, nk, d):
    qi = synth.qkvdo(seed, (B, H, nq, d), "bf16")
    ki = synth.qkvdo(seed + 1, (B, H, nk, d), "bf16", with_do=False)
    return {"q": qi["q"], "q_raw": qi["q_raw"], "do": qi["do"], "do_raw": qi["do_raw"],
            "k": ki["k"], "k_raw": ki["k_raw"], "v": ki["v"], "v_raw": ki["v_raw"]}


def _check_fwd(o, lse, o_r, lse_r):
    empty = np.isneginf(lse_r)
    assert np.array_equal(np.isneginf(lse), empty), "empty-row pattern of LSE"
    assert np.all(o[empty] == 0)
    live = ~empty
    assert_close(o[live], o_r[live], "bf16", "O")
    assert_close(lse[live], lse_r[live], "bf16", "LSE")


CASES = [
    # (B, H, Nq, Nk, d): queries after a cache, ragged; more queries than keys
    (2, 2, 200, 700, 64),
    (1, 3, 77, 1000, 128),
    (2, 2, 300, 130, 64),
    (1, 2, 129, 64, 128),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CASES)
def test_unequal_lengths_forward_and_backward(case, causal):
    E = _api()
    B, H, nq, nk, d = case
    seed = 6000 + nq + nk + d + causal
    _announce("qk fwd+bwd", case, "causal" if causal else "full", "seed", seed)
    inp = _inputs(seed, B, H, nq, nk, d)
    q, k, v, do = (upload(inp[x + "_raw"], "bf16") for x in ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(d)
    o, lse = E.attn_fwd_qk(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = E.attn_bwd_qk(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_r, lse_r = VL.forward_qk_batched(inp["q"], inp["k"], inp["v"], causal, scale)
    g_r = VL.backward_qk_batched(inp["q"], inp["k"], inp["v"], inp["do"], causal, scale)
    _check_fwd(download(o), download(lse), o_r, lse_r)
    empty = np.isneginf(lse_r)
    assert np.all(download(dq)[empty] == 0)
    assert_close(download(dq), g_r[0], "bf16", "dQ")
    assert_close(download(dk), g_r[1], "bf16", "dK")
    assert_close(download(dv), g_r[2], "bf16", "dV")


@pytest.mark.parametrize("splits", [1, 3, 8, 0])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,d", [(1, 128), (16, 64)])
def test_decode_split_kv(nq, d, causal, splits):
    E = _api()
    B, H, nk = 2, 4, 5000
    seed = 6100 + nq + d + causal
    _announce("decode", (B, H, nq, nk, d), "causal" if causal else "full", "splits", splits)
    inp = _inputs(seed, B, H, nq, nk, d)
    q, k, v = (upload(inp[x + "_raw"], "bf16") for x in ("q", "k", "v"))
    o, lse = E.attn_fwd_qk(q, k, v, causal=causal, num_splits=splits)
    torch.cuda.synchronize()
    o_r, lse_r = VL.forward_qk_batched(inp["q"], inp["k"], inp["v"], causal)
    _check_fwd(download(o), download(lse), o_r, lse_r)


DECODE_CASES = [
    # (B, H, Nq, Nk, d): one to four query rows (the vector-ALU decode kernel)
    (1, 3, 1, 1, 128),  # a single key
    (2, 2, 1, 63, 64),  # less than one load batch
    (1, 2, 2, 2, 128),  # as many queries as keys
    (2, 3, 3, 129, 128),  # ragged last chunk
    (1, 2, 4, 4, 64),
    (2, 2, 4, 1000, 64),
    (1, 4, 3, 4097, 128),
    (1, 2, 4, 3, 64),  # more query rows than keys: the matrix-core kernel (empty first row)
]


@pytest.mark.parametrize("splits", [1, 2, 0])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", DECODE_CASES)
def test_decode_kernel_rows_and_tails(case, causal, splits):
    E = _api()
    B, H, nq, nk, d = case
    seed = 6300 + 7 * nq + nk + d + causal
    _announce("decode kernel", case, "causal" if causal else "full", "splits", splits, "seed", seed)
    inp = _inputs(seed, B, H, nq, nk, d)
    q, k, v = (upload(inp[x + "_raw"], "bf16") for x in ("q", "k", "v"))
    o, lse = E.attn_fwd_qk(q, k, v, causal=causal, num_splits=splits)
    torch.cuda.synchronize()
    o_r, lse_r = VL.forward_qk_batched(inp["q"], inp["k"], inp["v"], causal)
    _check_fwd(download(o), download(lse), o_r, lse_r)


@pytest.mark.parametrize("scale", [-0.3, 0.02, 0.0])
def test_decode_kernel_scales(scale):
    # Negative, small and zero scales (the kernel multiplies the fp32 score by
    # scale * log2(e) before the max; zero gives the uniform average of V and
    # LSE = log Nk).
    E = _api()
    B, H, nq, nk, d = 2, 2, 2, 777, 128
    _announce("decode kernel scale", scale)
    inp = _inputs(6400, B, H, nq, nk, d)
    q, k, v = (upload(inp[x + "_raw"], "bf16") for x in ("q", "k", "v"))
    o, lse = E.attn_fwd_qk(q, k, v, causal=True, scale=scale, num_splits=0)
    torch.cuda.synchronize()
    o_r, lse_r = VL.forward_qk_batched(inp["q"], inp["k"], inp["v"], True, scale)
    _check_fwd(download(o), download(lse), o_r, lse_r)


def test_decode_kernel_many_heads_unsplit():
    # 1024 heads fill the chip without a split: every workgroup writes O and
    # LSE directly.
    E = _api()
    B, H, nq, nk, d = 16, 64, 1, 300, 64
    _announce("decode kernel many heads", (B, H, nq, nk, d))
    assert E.lib().attn_fwd_qk_workspace_bytes(B, H, nq, nk, d, E.ATTN_BF16, 0) == 0
    inp = _inputs(6500, B, H, nq, nk, d)
    q, k, v = (upload(inp[x + "_raw"], "bf16") for x in ("q", "k", "v"))
    o, lse = E.attn_fwd_qk(q, k, v, causal=False)
    torch.cuda.synchronize()
    o_r, lse_r = VL.forward_qk_batched(inp["q"], inp["k"], inp["v"], False)
    _check_fwd(download(o), download(lse), o_r, lse_r)


def _decode_setup(E, B, H, nq, nk, d, seed):
    inp = _inputs(seed, B, H, nq, nk, d)
    q, k, v = (upload(inp[x + "_raw"], "bf16") for x in ("q", "k", "v"))
    need = int(E.lib().attn_fwd_qk_workspace_bytes(B, H, nq, nk, d, E.ATTN_BF16, 0))
    assert need > 0
    return inp, q, k, v, need


def test_decode_kernel_deterministic():
    # The chunks' partials are merged in a fixed order: the result does not
    # depend on the workspace's earlier contents, and repeated calls give the
    # first call's bits.
    E = _api()
    B, H, nq, nk, d = 2, 3, 1, 3000, 128
    _announce("decode kernel determinism", (B, H, nq, nk, d))
    inp, q, k, v, need = _decode_setup(E, B, H, nq, nk, d, 6600)
    zero = torch.zeros(need, dtype=torch.uint8, device="cuda")
    o0, l0 = E.attn_fwd_qk(q, k, v, causal=True, num_splits=0, workspace=zero)
    g = torch.Generator(device="cuda").manual_seed(5)
    noise = torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda", generator=g)
    ones = torch.full((need,), 255, dtype=torch.uint8, device="cuda")
    for name, ws in (("random", noise), ("ones", ones)):
        o, l = E.attn_fwd_qk(q, k, v, causal=True, num_splits=0, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o, o0) and torch.equal(l, l0), name
    outs = [E.attn_fwd_qk(q, k, v, causal=True, num_splits=0, workspace=zero) for _ in range(40)]
    torch.cuda.synchronize()
    for i, (o, l) in enumerate(outs):
        assert torch.equal(o, o0) and torch.equal(l, l0), f"call {i}"
    o_r, lse_r = VL.forward_qk_batched(inp["q"], inp["k"], inp["v"], True)
    _check_fwd(download(o0), download(l0), o_r, lse_r)


def test_decode_kernel_many_heads_split_merged_separately():
    # More than 1024 heads with an explicit split (the automatic plan would
    # not split): 2080 workgroups of two chunks each.
    E = _api()
    B, H, nq, nk, d = 2, 520, 1, 600, 64
    _announce("decode kernel many heads split", (B, H, nq, nk, d))
    inp = _inputs(6800, B, H, nq, nk, d)
    q, k, v = (upload(inp[x + "_raw"], "bf16") for x in ("q", "k", "v"))
    o, lse = E.attn_fwd_qk(q, k, v, causal=False, num_splits=2)
    torch.cuda.synchronize()
    o_r, lse_r = VL.forward_qk_batched(inp["q"], inp["k"], inp["v"], False)
    _check_fwd(download(o), download(lse), o_r, lse_r)


def test_decode_kernel_graph_replays():
    # The decode kernel and the merge kernel captured once and replayed, with
    # eager calls on another workspace between the replays.
    E = _api()
    B, H, nq, nk, d = 1, 4, 2, 2500, 64
    _announce("decode kernel graph", (B, H, nq, nk, d))
    inp, q, k, v, need = _decode_setup(E, B, H, nq, nk, d, 6700)
    ws_e = torch.empty(need, dtype=torch.uint8, device="cuda")
    ref_o, ref_l = E.attn_fwd_qk(q, k, v, causal=True, num_splits=0, workspace=ws_e)
    torch.cuda.synchronize()
    ws_g = torch.empty(need, dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, nq), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        E.attn_fwd_qk(q, k, v, causal=True, num_splits=0, out=o, lse=lse, workspace=ws_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        E.attn_fwd_qk(q, k, v, causal=True, num_splits=0, out=o, lse=lse, workspace=ws_g)
    for i in range(4):
        o.zero_()
        lse.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l), f"replay {i}"
        E.attn_fwd_qk(q, k, v, causal=True, num_splits=0, workspace=ws_e)
        torch.cuda.synchronize()
    o_r, lse_r = VL.forward_qk_batched(inp["q"], inp["k"], inp["v"], True)
    _check_fwd(download(ref_o), download(ref_l), o_r, lse_r)


BENCH_DECODE = [
    # The benchmark's decode lines (causal, B=1 H=32): one query row over 4096,
    # 16384 and 65536 keys at d = 128, four rows over 16384, one at d = 64.
    (1, 32, 1, 4096, 128),
    (1, 32, 1, 16384, 128),
    (1, 32, 1, 65536, 128),
    (1, 32, 4, 16384, 128),
    (1, 32, 1, 16384, 64),
]


@pytest.mark.parametrize("case", BENCH_DECODE)
def test_decode_bench_shapes_every_output(case):
    # Every output row of each benchmark decode shape, in the launch
    # configurations the benchmark times (the automatic split and one pass).
    E = _api()
    B, H, nq, nk, d = case
    seed = 6900 + nq + d + nk // 1024
    _announce("decode bench shape", case, "seed", seed)
    inp = _inputs(seed, B, H, nq, nk, d)
    q, k, v = (upload(inp[x + "_raw"], "bf16") for x in ("q", "k", "v"))
    o_r, lse_r = VL.forward_qk_batched(inp["q"], inp["k"], inp["v"], True)
    for splits in (0, 1):
        o, lse = E.attn_fwd_qk(q, k, v, causal=True, num_splits=splits)
        torch.cuda.synchronize()
        _check_fwd(download(o), download(lse), o_r, lse_r)


def test_long_decode_auto_split():
    # Four queries after 65532 cached tokens, one head group, automatic split.
    E = _api()
    B, H, nq, nk, d = 1, 4, 4, 65536, 128
    _announce("decode long", (B, H, nq, nk, d))
    inp = _inputs(6200, B, H, nq, nk, d)
    q, k, v = (upload(inp[x + "_raw"], "bf16") for x in ("q", "k", "v"))
    assert E.lib().attn_fwd_qk_workspace_bytes(B, H, nq, nk, d, E.ATTN_BF16, 0) > 0
    o, lse = E.attn_fwd_qk(q, k, v, causal=True, num_splits=0)
    torch.cuda.synchronize()
    o_r, lse_r = VL.forward_qk_batched(inp["q"], inp["k"], inp["v"], True)
    _check_fwd(download(o), download(lse), o_r, lse_r)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_equal_lengths_match_square_path_bitwise(d, causal):
    # Nq == Nk without a split does the square path's arithmetic in its order.
    # Exception: at d = 64 the square dense backward computes dK and dV with
    # the single-role kernel (attn_bwd_kv64.hip), the other paths with the
    # paired-wave kernel.  The two add the same terms in the same order except
    # in blocks that take the hi + lo split (a block's lo terms come before its
    # hi terms in one, after them in the other), so there dK and dV agree to
    # the bf16 rounding of the outputs.
    E = _api()
    B, H, n = 2, 2, 333
    _announce("qk == square", d, "causal" if causal else "full")
    inp = synth.qkvdo(6300 + d + causal, (B, H, n, d), "bf16")
    q, k, v, do = (upload(inp[x + "_raw"], "bf16") for x in ("q", "k", "v", "do"))
    o1, l1 = E.attn_fwd_qk(q, k, v, causal=causal)
    g1 = E.attn_bwd_qk(q, k, v, o1, do, l1, causal=causal)
    o2, l2 = E.attn_fwd(q, k, v, causal=causal)
    g2 = E.attn_bwd(q, k, v, o2, do, l2, causal=causal)
    torch.cuda.synchronize()
    for name, a, b in zip(("O", "LSE", "dQ", "dK", "dV"), (o1, l1) + tuple(g1), (o2, l2) + tuple(g2)):
        if d == 64 and name in ("dK", "dV"):
            diff = (a.float() - b.float()).abs()
            assert float((diff / b.float().abs().clamp_min(1.0)).max()) <= 2.0**-7, name
        else:
            assert torch.equal(a, b), name


def _dsum_bytes(B, H, nq):
    return -(-(B * H * nq * 4) // 256) * 256


# (B, H, Nq, Nk, d): decoding (one query), a ragged last chunk, more queries
# than keys (rows that see no key of some chunks, or none at all).
SPLIT_CASES = [(2, 4, 1, 5000, 128), (1, 2, 300, 1030, 64), (1, 1, 700, 600, 128), (2, 2, 64, 4096, 64)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", SPLIT_CASES)
def test_backward_with_dq_split_over_keys(case, causal):
    # Few (head, query block) workgroups: the library splits the dQ pass over
    # key chunks and sums the fp32 partials; the workspace holds them.
    E = _api()
    B, H, nq, nk, d = case
    assert E.lib().attn_bwd_qk_workspace_bytes(B, H, nq, nk, d, E.ATTN_BF16) > _dsum_bytes(B, H, nq)
    seed = 6400 + nq + nk + d + causal
    _announce("qk bwd, dQ split", case, "causal" if causal else "full", "seed", seed)
    inp = _inputs(seed, B, H, nq, nk, d)
    q, k, v, do = (upload(inp[x + "_raw"], "bf16") for x in ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(d)
    o, lse = E.attn_fwd_qk(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = E.attn_bwd_qk(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_r, lse_r = VL.forward_qk_batched(inp["q"], inp["k"], inp["v"], causal, scale)
    g_r = VL.backward_qk_batched(inp["q"], inp["k"], inp["v"], inp["do"], causal, scale)
    _check_fwd(download(o), download(lse), o_r, lse_r)
    empty = np.isneginf(lse_r)
    assert np.all(download(dq)[empty] == 0)
    assert_close(download(dq), g_r[0], "bf16", "dQ")
    assert_close(download(dk), g_r[1], "bf16", "dK")
    assert_close(download(dv), g_r[2], "bf16", "dV")


@pytest.mark.parametrize("causal", [False, True])
def test_chunked_prefill_forward_and_sampled_backward(causal):
    # 1024 queries after 7168 cached tokens, 16 heads, d = 128: the forward
    # (four key chunks) on every head, the backward (the dQ pass in four key
    # chunks of 2048) on four whole heads, against the oracle.
    E = _api()
    B, H, nq, nk, d = 1, 16, 1024, 8192, 128
    assert E.lib().attn_bwd_qk_workspace_bytes(B, H, nq, nk, d, E.ATTN_BF16) == (
        _dsum_bytes(B, H, nq) + 4 * B * H * nq * d * 4)
    _announce("chunked prefill bwd", (B, H, nq, nk, d), "causal" if causal else "full")
    inp = _inputs(6500 + causal, B, H, nq, nk, d)
    q, k, v, do = (upload(inp[x + "_raw"], "bf16") for x in ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(d)
    o, lse = E.attn_fwd_qk(q, k, v, causal=causal, scale=scale, num_splits=0)
    dq, dk, dv = E.attn_bwd_qk(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_r, lse_r = VL.forward_qk_batched(inp["q"], inp["k"], inp["v"], causal, scale)
    _check_fwd(download(o), download(lse), o_r, lse_r)
    got = [download(t) for t in (dq, dk, dv)]
    for h in synth.sample_pairs(6510 + causal, H, 1, 4)[:, 0]:
        g_r = VL.backward_qk(inp["q"][0, h], inp["k"][0, h], inp["v"][0, h], inp["do"][0, h], causal, scale)
        for name, g, r in zip(("dQ", "dK", "dV"), got, g_r):
            assert_close(g[0, h], r, "bf16", f"{name} (head {h})")
