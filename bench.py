"""Throughput of the fused attention path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic bf16
inputs at B=4, H=16, N=4096, d=128 (the d = 128, N >= 4096 shape the
performance target is stated for): for the full mask and for the causal mask,
the forward kernel (O, LSE), then the backward as attn_bwd runs it: the dQ
pass, which also forms D = rowsum(dO * O), then the dK/dV pass.  Inputs are
resident in HBM before the timed region starts.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
       (without --no-cpu the line also carries two CPU references on bounded
       samples of the workload: the float64 oracle, cpu_baseline, and the
       cache-blocked CPU implementation of libattn_cpu.so, cpu_flash)
       python bench.py --sweep           (one JSON line per N, d, mask, pass)
       python bench.py --blocksparse     (block-sparse vs dense, one JSON line
                                          per block density and mask)
       python bench.py --decode          (unequal lengths: split-K/V decoding
                                          and chunked prefill, one JSON line each)
       python bench.py --dropout         (fused dropout against the plain path,
                                          one JSON line per mask)
       python bench.py --profile-pass    (one step plus a plain copy of known
                                          size, for hardware-counter runs)

Prints one JSON line.  FLOP convention: forward 4*B*H*N^2*d (two N x N x d
products), halved under the causal mask; backward 2.5x forward (five
products, one of them the recomputation of Q K^T).  Peak: MI355X dense bf16
matrix throughput, 2516.6 TFLOP/s (256 CUs x 2.4 GHz x 4096 flop/clk/CU).
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0
METRIC = "attention fwd/bwd TFLOP/s at N=1K–64K, d=64/128; % of bf16 MFMA peak"
KERNEL_SOURCES = {
    "fwd": "exact_io_aware_05_amd/csrc/attn_fwd_bf16.hip",
    "dkdv": "exact_io_aware_05_amd/csrc/attn_bwd_bf16.hip",
    "dq": "exact_io_aware_05_amd/csrc/attn_bwd_bf16.hip",
}
KERNEL_NAMES = {  # substrings of the compiled kernel symbols, as rocprofv3 lists them
    "fwd": "fwd_bf16_kernel",
    "dkdv": "bwd_kv_kernel",
    "dq": "bwd_q_kernel",
}


def fwd_flops(bh, n, d, causal):
    f = 4.0 * bh * n * n * d
    return f / 2 if causal else f


def phase_flops(phase, bh, n, d, causal):
    """Algorithmic flops of one launch of a phase (sums to fwd + 2.5 fwd)."""
    g = 2.0 * bh * n * n * d / (2 if causal else 1)  # one N x N x d product
    return {"fwd": 2 * g, "dkdv": 4 * g, "dq": 1 * g, "dsum": 0.0}[phase]


def phase_bytes(phase, bh, n, d):
    """Minimum HBM bytes of one launch of a phase (bf16 tensors, fp32 rows)."""
    t = 2.0 * bh * n * d  # one bf16 [B,H,N,d] tensor
    r = 4.0 * bh * n  # one fp32 [B,H,N] vector
    return {
        "fwd": 4 * t + r,  # read Q, K, V; write O, LSE
        "dsum": 2 * t + r,  # read O, dO; write D
        "dkdv": 6 * t + 2 * r,  # read Q, K, V, dO, LSE, D; write dK, dV
        "dq": 6 * t + 2 * r,  # read Q, K, V, O, dO, LSE; write dQ, D
    }[phase]


def source_hash(phase):
    with open(os.path.join(ROOT, KERNEL_SOURCES[phase]), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(phase, workload, masks):
    """HBM bytes per launch from committed counter summaries, if still current."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            data = json.load(f)
        entry = data[workload][phase + ("_causal" if masks else "")]
        if entry.get("source_sha256_16") != source_hash(phase):
            return None
        return entry["bytes_per_launch"]
    except (KeyError, ValueError, TypeError):
        return None


def cpu_baseline(shape, budget_s=12.0, max_heads=256):
    """The float64 oracle on a bounded sample of the same workload (host cores)."""
    from threadpoolctl import threadpool_info

    import synth
    from oracle import attention as A

    b, h, n, d = shape
    inp = synth.qkvdo(3, (1, 2, n, d), "bf16")  # two heads of the same shape and distribution
    scale = 1.0 / math.sqrt(d)
    flops = 0.0
    heads = 0
    t0 = time.perf_counter()
    while heads < max_heads and (time.perf_counter() - t0) < budget_s:
        causal = heads % 2 == 1
        hd = heads % 2
        q, k, v, do = (inp[x][0, hd] for x in ("q", "k", "v", "do"))
        A.forward_head(q, k, v, causal, scale)
        A.backward_head(q, k, v, do, causal, scale)
        flops += 3.5 * fwd_flops(1, n, d, causal)
        heads += 1
    dt = time.perf_counter() - t0
    threads = 1
    blas = {}
    for info in threadpool_info():
        if info.get("user_api") == "blas":
            threads = max(threads, int(info.get("num_threads", 1)))
            blas = {"library": info.get("internal_api"), "version": info.get("version"),
                    "threads": int(info.get("num_threads", 1)),
                    "file": os.path.basename(info.get("filepath") or "")}
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{heads} (batch, head) slices of N={n} d={d}, alternating full/causal mask, "
        f"forward + backward in float64 ({dt:.1f} s, {flops / 1e9:.0f} GFLOP by the same convention)",
        "cpu_model": cpu_model(),
        "host_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "blas": blas,
        "long_context_rows": long_context_rows_baseline(),
    }


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def long_context_rows_baseline():
    """The oracle's row-restricted forms on the N = 65536 workload (B=1 H=8
    d=64, causal): O, LSE and dQ of its 512 seeded query rows, and the
    per-row statistics pass (LSE and D of whole rows, which the key-row
    gradients need for every row of a head) on one 1024-row block.  Reported
    as measured rows per second; nothing is extrapolated."""
    import synth
    from oracle import attention as A

    w = synth.WORKLOADS["long_n65536_d64_causal"]
    inp = synth.qkvdo(w.seed, w.shape, w.dtype)
    bh = w.b * w.h
    flat = {x: inp[x].reshape(bh, w.n, w.d) for x in ("q", "k", "v", "do")}
    scale = 1.0 / math.sqrt(w.d)
    pairs = synth.sample_pairs(w.seed + 1, bh, w.n, 512)
    t0 = time.perf_counter()
    for hd in np.unique(pairs[:, 0]):
        rows = pairs[pairs[:, 0] == hd, 1]
        a = [flat[x][hd] for x in ("q", "k", "v", "do")]
        A.forward_rows(a[0], a[1], a[2], rows, True, scale)
        A.backward_query_rows(a[0], a[1], a[2], a[3], rows, True, scale)
    t_q = time.perf_counter() - t0
    # One block of whole rows (the last 256 rows of head 0, the longest
    # causal rows): LSE, and D_i with dQ (backward_query_rows forms P, dP and
    # D of its rows), the work the statistics pass does per block plus dQ.
    a = [flat[x][0] for x in ("q", "k", "v", "do")]
    rows = np.arange(w.n - 256, w.n)
    t0 = time.perf_counter()
    A.forward_rows(a[0], a[1], a[2], rows, True, scale)
    A.backward_query_rows(a[0], a[1], a[2], a[3], rows, True, scale)
    t_s = time.perf_counter() - t0
    return {
        "workload": "B=1 H=8 N=65536 d=64 causal, float64 oracle",
        "query_rows": 512,
        "query_rows_s": round(t_q, 2),
        "query_rows_per_s": round(512 / t_q, 1),
        "what": "O, LSE and dQ of the 512 seeded query rows; O, LSE, D and dQ of the last 256 rows of head 0 "
        "(the per-block work of the statistics pass that the key rows' dK, dV need over every row of a head)",
        "stat_rows": 256,
        "stat_rows_s": round(t_s, 2),
        "stat_rows_per_s": round(256 / t_s, 1),
    }


def cpu_flash(shape, budget_s=8.0, max_heads=64):
    """The cache-blocked multi-core CPU form of the method (libattn_cpu.so) on
    a bounded sample of the same workload: (batch, head) slices of the same
    shape, alternating full/causal mask, forward + backward, all host threads."""
    import synth
    from exact_io_aware_05_amd import cpu as C

    b, h, n, d = shape
    inp = synth.qkvdo(3, (1, 2, n, d), "bf16")
    q, k, v, do = (inp[x].astype(np.float32) for x in ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(d)
    C.attn_cpu_fwd(q[:, :1, :64], k[:, :1, :64], v[:, :1, :64])  # load the library, start the threads
    flops, heads = 0.0, 0
    t0 = time.perf_counter()
    while heads < max_heads and (time.perf_counter() - t0) < budget_s:
        causal = heads % 2 == 1
        sl = slice(heads % 2, heads % 2 + 1)
        o, lse = C.attn_cpu_fwd(q[:, sl], k[:, sl], v[:, sl], causal, scale)
        C.attn_cpu_bwd(q[:, sl], k[:, sl], v[:, sl], o, do[:, sl], lse, causal, scale)
        flops += 3.5 * fwd_flops(1, n, d, causal)
        heads += 1
    dt = time.perf_counter() - t0
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(os.environ.get("OMP_NUM_THREADS") or len(os.sched_getaffinity(0))),
        "kind": "cache-blocked CPU implementation (fp32, OpenMP)",
        "sample": f"{heads} (batch, head) slices of N={n} d={d}, alternating full/causal mask, "
        f"forward + backward ({dt:.1f} s)",
    }


class Buffers:
    def __init__(self, torch, shape, causal, seed=3):
        import synth

        inp = synth.qkvdo(seed, shape, "bf16")
        dev = "cuda"

        def up(raw):
            return torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16).to(dev)

        self.q, self.k, self.v, self.do = (up(inp[x + "_raw"]) for x in ("q", "k", "v", "do"))
        b, h, n, d = shape
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((b, h, n), dtype=torch.float32, device=dev)
        self.dsum = torch.empty((b, h, n), dtype=torch.float32, device=dev)
        self.dq = torch.empty_like(self.q)
        self.dk = torch.empty_like(self.k)
        self.dv = torch.empty_like(self.v)
        self.causal = causal
        self.scale = 1.0 / math.sqrt(d)


def run_step(E, bufs, events=None):
    """One step: for each mask, the forward, then the backward as attn_bwd runs
    it: dQ with D formed inside the dQ pass, then dK/dV."""
    k = 0
    for B in bufs:
        if events is not None:
            events[k].record()
        E.attn_fwd(B.q, B.k, B.v, B.causal, B.scale, out=B.o, lse=B.lse)
        if events is not None:
            events[k + 1].record()
        E.attn_bwd_dq_dsum(B.q, B.k, B.v, B.o, B.do, B.lse, B.causal, B.scale, dsum=B.dsum, dq=B.dq)
        if events is not None:
            events[k + 2].record()
        E.attn_bwd_dkdv(B.q, B.k, B.v, B.do, B.lse, B.dsum, B.causal, B.scale, dk=B.dk, dv=B.dv)
        if events is not None:
            events[k + 3].record()
        k += 4


PHASES = ["fwd", "dq", "dkdv"]
EVENTS_PER_MASK = len(PHASES) + 1


def measure(torch, E, shape, steps, warmup):
    bufs = [Buffers(torch, shape, False), Buffers(torch, shape, True)]
    for _ in range(warmup):
        run_step(E, bufs)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * EVENTS_PER_MASK)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        run_step(E, bufs, ev[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    per = {}
    for mi, mask in enumerate(("full", "causal")):
        for pi, ph in enumerate(PHASES):
            a = EVENTS_PER_MASK * mi + pi
            ms = [ev[s][a].elapsed_time(ev[s][a + 1]) for s in range(steps)]
            per[(mask, ph)] = float(np.mean(ms))
    return (t1 - t0) * 1e3 / steps, per


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--profile-pass", action="store_true")
    ap.add_argument("--profile-pass-d64", action="store_true",
                    help="one causal step at B=8 H=16 N=2048 d=64 and one causal forward at B=8 H=12 N=1024 d=64")
    ap.add_argument("--blocksparse", action="store_true")
    ap.add_argument("--decode", action="store_true")
    ap.add_argument("--dropout", action="store_true")
    ap.add_argument("--window", action="store_true")
    ap.add_argument("--probes", action="store_true", help="diagnostic microbenchmarks (libattn_probe.so)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(
            f"bench.py: --gpus {args.gpus} requested; the library runs on one GPU only "
            "(the kernels work on one device's share and there is no multi-GPU path)",
            file=sys.stderr,
        )
        sys.exit(2)

    import torch

    import exact_io_aware_05_amd as E

    E.lib()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)

    if args.profile_pass:
        shape = (4, 16, 4096, 128)
        bufs = [Buffers(torch, shape, False), Buffers(torch, shape, True)]
        run_step(E, bufs)
        torch.cuda.synchronize()
        src = torch.empty(256 * 2**20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)  # plain copy of 256 MiB: 256 MiB read + 256 MiB written
        torch.cuda.synchronize()
        print(json.dumps({"profile_pass": "done", "copy_bytes_each_way": 256 * 2**20}), flush=True)
        return

    if args.profile_pass_d64:
        # For counter passes of the d = 64 kernels: a warm-up step, then the
        # profiled one (the same launches as the bench's own timing of these
        # workloads).
        b4 = [Buffers(torch, (8, 16, 2048, 64), True)]
        b2 = Buffers(torch, (8, 12, 1024, 64), True)
        for _ in range(2):
            run_step(E, b4)
            E.attn_fwd(b2.q, b2.k, b2.v, True, b2.scale, out=b2.o, lse=b2.lse)
        torch.cuda.synchronize()
        print(json.dumps({"profile_pass_d64": "done"}), flush=True)
        return

    if args.sweep:
        sweep(torch, E, args.steps, args.warmup)
        return

    if args.probes:
        probes(torch)
        return

    if args.blocksparse:
        blocksparse(torch, E, args.steps, args.warmup)
        return

    if args.decode:
        decode(torch, E, args.steps, args.warmup)
        return

    if args.dropout:
        dropout(torch, E, args.steps, args.warmup)
        return

    if args.window:
        window(torch, E, args.steps, args.warmup)
        return

    shape = (4, 16, 4096, 128)
    b, h, n, d = shape
    bh = b * h
    ms_step, per = measure(torch, E, shape, args.steps, args.warmup)
    total_flops = sum(3.5 * fwd_flops(bh, n, d, c) for c in (False, True))
    value = total_flops / (ms_step * 1e-3) / 1e12

    breakdown = {}
    for mask in ("full", "causal"):
        causal = mask == "causal"
        fwd_ms = per[(mask, "fwd")]
        bwd_ms = per[(mask, "dq")] + per[(mask, "dkdv")]
        ff = fwd_flops(bh, n, d, causal)
        breakdown[mask] = {
            "fwd_ms": round(fwd_ms, 4),
            "fwd_tflops": round(ff / fwd_ms / 1e9, 1),
            "fwd_frac_peak": round(ff / fwd_ms / 1e9 / PEAK_BF16_TFLOPS, 4),
            "bwd_ms": round(bwd_ms, 4),
            "bwd_tflops": round(2.5 * ff / bwd_ms / 1e9, 1),
            "bwd_frac_peak": round(2.5 * ff / bwd_ms / 1e9 / PEAK_BF16_TFLOPS, 4),
            "kernel_ms": {ph: round(per[(mask, ph)], 4) for ph in PHASES},
        }

    # Dominant kernel: the single launch with the largest average duration.
    (dmask, dph), dms = max(per.items(), key=lambda kv: kv[1])
    causal = dmask == "causal"
    fl = phase_flops(dph, bh, n, d, causal)
    achieved = fl / (dms * 1e-3) / 1e12
    traffic = load_traffic(dph, "n4096_d128", causal)
    roofline = {
        "bound": "mfma",
        "achieved": round(achieved, 1),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": traffic,
        "kernel": KERNEL_NAMES[dph] + (" (causal)" if causal else " (full mask)"),
        "kernel_ms": round(dms, 4),
        "algorithmic_flops_per_launch": fl,
        "min_hbm_bytes_per_launch": phase_bytes(dph, bh, n, d),
    }

    configs = config_entries(torch, E)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "fused attention forward + backward, B=4 H=16 N=4096 d=128, full and causal mask",
            "B": b,
            "H": h,
            "N": n,
            "d": d,
            "masks": ["full", "causal"],
            "parallelism": "none (1 GPU)",
        },
        "roofline": roofline,
        "breakdown": breakdown,
        "configs": configs,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(shape)
        out["cpu_flash"] = cpu_flash(shape)
    print(json.dumps(out), flush=True)


PEAK_FP32_TFLOPS = 157.3


def probes(torch):
    """Diagnostic microbenchmarks, one JSON line each: fp32 atomic adds of a dQ
    accumulated by key blocks (and plain stores of the same tiles) at the
    B=8 H=16 N=2048 d=64 and B=4 H=16 N=4096 d=128 shapes, the instruction-mix
    cycles at one and two waves per SIMD, the MFMA rate and clock under load,
    and the read bandwidth of a plain streaming kernel over 1 GiB."""
    from exact_io_aware_05_amd import diag

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for d, heads, n in ((64, 128, 2048), (128, 64, 4096)):
        for causal in (True, False):
            for atomic in (True, False):
                r = diag.atomic_dq(d, heads, n, causal, atomic)
                print(json.dumps({"probe": "atomic_dq", "d": d, "heads": heads, "n": n, "causal": causal,
                                  "op": "fp32 atomic add" if atomic else "plain store",
                                  "ms": round(r["ms"], 4), "GB_per_s": round(r["GB_per_s"], 1),
                                  "bytes": r["bytes"], "mismatches": r["mismatches"]}), flush=True)
    for waves in (1, 2):
        for mix, name in diag.MIXES.items():
            r = diag.issue_mix(mix, waves, cus)
            print(json.dumps({"probe": "issue_mix", "mix": name, "waves_per_simd": waves,
                              "mean_cycles_per_iter": round(r["mean_cycles"], 1),
                              "max_cycles_per_iter": round(r["max_cycles"], 1)}), flush=True)
    r = diag.mfma_rate(cus)
    print(json.dumps({"probe": "mfma_rate", "cus": cus, "tflops": round(r["tflops"], 1), "ghz": round(r["ghz"], 3),
                      "frac_of_2516.6": round(r["tflops"] / 2516.6, 3)}), flush=True)
    for wgs_per_cu in (1, 2, 4, 8):
        for unroll in (4, 8, 16):
            r = diag.read_bw(1 << 30, wgs_per_cu * cus, unroll)
            print(json.dumps({"probe": "read_bw", "bytes": 1 << 30, "workgroups": wgs_per_cu * cus,
                              "loads_in_flight_per_thread": unroll, "ms": round(r["ms"], 4),
                              "GB_per_s": round(r["GB_per_s"], 1), "frac_of_8000": round(r["GB_per_s"] / 8000, 4)}),
                  flush=True)


def _upload(torch, inp, dtype):
    if dtype == "bf16":
        return [torch.from_numpy(inp[x + "_raw"].view(np.int16)).view(torch.bfloat16).cuda()
                for x in ("q", "k", "v", "do")]
    return [torch.from_numpy(inp[x + "_raw"]).cuda() for x in ("q", "k", "v", "do")]


def config_entries(torch, E, reps=20):
    """Each measured workload at its own shape, outside the timed step: HIP
    events on the library's stream around `reps` back-to-back calls of each
    pass (after 3 warm-up calls); TFLOP/s by the step's convention and as a
    fraction of the peak of the arithmetic (fp32 vector peak for the float32
    workload)."""
    import synth

    out = {}
    for name in ("fp32_n256_d64", "gpt2s_n1024_d64_causal", "bwd_n2048_d64_causal", "long_n65536_d64_causal"):
        w = synth.WORKLOADS[name]
        inp = synth.qkvdo(w.seed, w.shape, w.dtype)
        q, k, v, do = _upload(torch, inp, w.dtype)
        del inp
        scale = 1.0 / math.sqrt(w.d)
        o, lse = E.attn_fwd(q, k, v, causal=w.causal, scale=scale)
        ws = torch.empty(E.attn_bwd_workspace_bytes(w.b, w.h, w.n, w.d, E.ATTN_BF16 if w.dtype == "bf16"
                                                    else E.ATTN_FP32), dtype=torch.uint8, device="cuda")
        grads = tuple(torch.empty_like(q) for _ in range(3))
        n_rep = reps if w.n <= 8192 else 3
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
        ff = fwd_flops(w.b * w.h, w.n, w.d, w.causal)
        t_f = _time_ms(torch, lambda: E.attn_fwd(q, k, v, causal=w.causal, scale=scale, out=o, lse=lse), n_rep, 3)
        e = {"shape": list(w.shape), "dtype": w.dtype, "mask": "causal" if w.causal else "full",
             "fwd_ms": round(t_f, 4), "fwd_tflops": round(ff / t_f / 1e9, 2),
             "fwd_frac_peak": round(ff / t_f / 1e9 / peak, 4),
             "peak_tflops": peak}
        if "bwd" in w.passes:
            t_b = _time_ms(torch, lambda: E.attn_bwd(q, k, v, o, do, lse, causal=w.causal, scale=scale,
                                                     workspace=ws, grads=grads), n_rep, 3)
            e.update({"bwd_ms": round(t_b, 4), "bwd_tflops": round(2.5 * ff / t_b / 1e9, 2),
                      "bwd_frac_peak": round(2.5 * ff / t_b / 1e9 / peak, 4)})
        out[name] = e
        del q, k, v, do, o, lse, ws, grads
        torch.cuda.empty_cache()
    return out


def sweep(torch, E, steps, warmup):
    """N in 1K..64K, d in {64, 128}, both masks: forward and backward TFLOP/s."""
    tokens = 16384
    for d in (64, 128):
        hh = 2048 // d
        for n in (1024, 2048, 4096, 8192, 16384, 32768, 65536):
            b = max(1, tokens // n)
            shape = (b, hh, n, d)
            bh = b * hh
            ms_step, per = measure(torch, E, shape, steps, warmup)
            for mask in ("full", "causal"):
                causal = mask == "causal"
                ff = fwd_flops(bh, n, d, causal)
                fwd_ms = per[(mask, "fwd")]
                bwd_ms = per[(mask, "dq")] + per[(mask, "dkdv")]
                print(
                    json.dumps(
                        {
                            "B": b, "H": hh, "N": n, "d": d, "mask": mask,
                            "fwd_ms": round(fwd_ms, 4),
                            "fwd_tflops": round(ff / fwd_ms / 1e9, 1),
                            "fwd_frac_peak": round(ff / fwd_ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                            "bwd_ms": round(bwd_ms, 4),
                            "bwd_tflops": round(2.5 * ff / bwd_ms / 1e9, 1),
                            "bwd_frac_peak": round(2.5 * ff / bwd_ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                            "kernel_ms": {ph: round(per[(mask, ph)], 4) for ph in PHASES},
                        }
                    ),
                    flush=True,
                )
            torch.cuda.empty_cache()



def allowed_pairs(mask, n, block, causal):
    """Number of (query, key) pairs a block mask (and the causal mask) allows."""
    idx = np.arange(n) // block
    total = 0
    for qb in range(mask.shape[0]):
        rows = np.arange(qb * block, min(n, (qb + 1) * block))
        cols = np.nonzero(mask[qb][idx])[0]
        if causal:
            total += int(np.sum(cols[None, :] <= rows[:, None]))
        else:
            total += len(rows) * len(cols)
    return total


def blocksparse(torch, E, steps, warmup):
    """Block-sparse forward + backward against dense at B=4 H=16 N=4096 d=128:
    random 128 x 128 block masks (the diagonal always kept) at several
    densities.  TFLOP/s counts only the allowed score entries (4 d flops per
    entry forward, 2.5x that backward)."""
    import synth

    b, h, n, d = 4, 16, 4096, 128
    bh = b * h
    nb = n // E.SPARSE_BLOCK
    g = torch.Generator(device="cuda").manual_seed(11)
    q, k, v, do = (torch.randn(b, h, n, d, device="cuda", generator=g).to(torch.bfloat16) for _ in range(4))
    ws = torch.empty(E.attn_bwd_workspace_bytes(b, h, n, d, E.ATTN_BF16), dtype=torch.uint8, device="cuda")
    for causal in (False, True):
        dense = None
        for density in (1.0, 0.5, 0.25):
            mask = synth.block_mask(5000 + int(100 * density), nb, density)
            mask[np.arange(nb), np.arange(nb)] = 1
            m = torch.from_numpy(mask).cuda()
            pairs = allowed_pairs(mask, n, E.SPARSE_BLOCK, causal) * bh

            def fwd():
                return E.attn_fwd_blocksparse(q, k, v, m, causal=causal)

            def bwd(o, lse):
                E.attn_bwd_blocksparse(q, k, v, o, do, lse, m, causal=causal, workspace=ws)

            o, lse = fwd()
            for _ in range(warmup):
                fwd()
                bwd(o, lse)
            torch.cuda.synchronize()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * steps)]
            for s_ in range(steps):
                ev[3 * s_].record()
                fwd()
                ev[3 * s_ + 1].record()
                bwd(o, lse)
                ev[3 * s_ + 2].record()
            torch.cuda.synchronize()
            fwd_ms = float(np.mean([ev[3 * i].elapsed_time(ev[3 * i + 1]) for i in range(steps)]))
            bwd_ms = float(np.mean([ev[3 * i + 1].elapsed_time(ev[3 * i + 2]) for i in range(steps)]))
            if density == 1.0:
                dense = (fwd_ms, bwd_ms)
            ff = 4.0 * d * pairs
            print(json.dumps({
                "blocksparse": True, "B": b, "H": h, "N": n, "d": d, "mask": "causal" if causal else "full",
                "block": E.SPARSE_BLOCK, "density": round(float(mask.mean()), 4),
                "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
                "fwd_tflops": round(ff / fwd_ms / 1e9, 1), "bwd_tflops": round(2.5 * ff / bwd_ms / 1e9, 1),
                "speedup_vs_dense": round((dense[0] + dense[1]) / (fwd_ms + bwd_ms), 3),
            }), flush=True)



def _time_ms(torch, fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _time_graph_ms(torch, fn, steps, warmup):
    """Per-call time of `steps` calls captured in one HIP graph and replayed
    (no host work between the calls): for calls short enough that Python's
    own per-call overhead would otherwise leave the GPU idle between them."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(steps):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def dropout(torch, E, steps, warmup):
    """Fused dropout against the plain path at B=4 H=16 N=4096 d=128, bf16:
    forward and whole backward (D, dK/dV, dQ) per mask, p = 0.1, TFLOP/s by
    the usual convention (the generator's work is not counted)."""
    shape = (4, 16, 4096, 128)
    b, h, n, d = shape
    g = torch.Generator(device="cuda").manual_seed(17)
    q, k, v, do = (torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16) for _ in range(4))
    ws = torch.empty(max(E.attn_bwd_workspace_bytes(b, h, n, d, E.ATTN_BF16), 256), dtype=torch.uint8, device="cuda")
    grads = tuple(torch.empty_like(q) for _ in range(3))
    for causal in (False, True):
        f = fwd_flops(b * h, n, d, causal)
        o, lse = E.attn_fwd(q, k, v, causal=causal)
        t_fwd = _time_ms(torch, lambda: E.attn_fwd(q, k, v, causal=causal, out=o, lse=lse), steps, warmup)
        t_bwd = _time_ms(torch, lambda: E.attn_bwd(q, k, v, o, do, lse, causal=causal, workspace=ws, grads=grads),
                         steps, warmup)
        od, lsed = E.attn_fwd_dropout(q, k, v, 0.1, 1234, 0, causal=causal)
        t_fwd_d = _time_ms(torch, lambda: E.attn_fwd_dropout(q, k, v, 0.1, 1234, 0, causal=causal, out=od, lse=lsed),
                           steps, warmup)
        t_bwd_d = _time_ms(torch, lambda: E.attn_bwd_dropout(q, k, v, od, do, lsed, 0.1, 1234, 0, causal=causal,
                                                             workspace=ws, grads=grads), steps, warmup)
        print(json.dumps({
            "mode": "dropout", "mask": "causal" if causal else "full", "B": b, "H": h, "N": n, "d": d, "p": 0.1,
            "fwd_ms": round(t_fwd_d, 4), "fwd_tflops": round(f / t_fwd_d / 1e9, 1),
            "bwd_ms": round(t_bwd_d, 4), "bwd_tflops": round(2.5 * f / t_bwd_d / 1e9, 1),
            "plain_fwd_ms": round(t_fwd, 4), "plain_bwd_ms": round(t_bwd, 4),
            "fwd_cost": round(t_fwd_d / t_fwd, 3), "bwd_cost": round(t_bwd_d / t_bwd, 3),
        }), flush=True)


def window(torch, E, steps, warmup):
    """Causal sliding window against the plain causal mask, bf16, d = 128:
    forward and whole backward at N = 4096 (B=4 H=16) and N = 16384 (B=1
    H=16) for windows of 256, 1024 and 4096 keys.  TFLOP/s count the products
    of the attended (query, key) pairs only: 4 d per pair forward, 2.5 times
    that backward."""
    for shape in ((4, 16, 4096, 128), (1, 16, 16384, 128)):
        b, h, n, d = shape
        g = torch.Generator(device="cuda").manual_seed(19)
        q, k, v, do = (torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16) for _ in range(4))
        ws = torch.empty(max(E.attn_bwd_workspace_bytes(b, h, n, d, E.ATTN_BF16), 256), dtype=torch.uint8,
                         device="cuda")
        grads = tuple(torch.empty_like(q) for _ in range(3))
        o, lse = E.attn_fwd(q, k, v, causal=True)
        t_fwd_c = _time_ms(torch, lambda: E.attn_fwd(q, k, v, causal=True, out=o, lse=lse), steps, warmup)
        t_bwd_c = _time_ms(torch, lambda: E.attn_bwd(q, k, v, o, do, lse, causal=True, workspace=ws, grads=grads),
                           steps, warmup)
        for win in (256, 1024, 4096):
            if win >= n:
                continue
            pairs = sum(min(i + 1, win) for i in range(n))
            f = 4.0 * d * pairs * b * h
            ow, lw = E.attn_fwd_window(q, k, v, win)
            t_fwd = _time_ms(torch, lambda: E.attn_fwd_window(q, k, v, win, out=ow, lse=lw), steps, warmup)
            t_bwd = _time_ms(torch, lambda: E.attn_bwd_window(q, k, v, ow, do, lw, win, workspace=ws, grads=grads),
                             steps, warmup)
            print(json.dumps({
                "mode": "window", "B": b, "H": h, "N": n, "d": d, "window": win,
                "fwd_ms": round(t_fwd, 4), "fwd_tflops": round(f / t_fwd / 1e9, 1),
                "fwd_frac_peak": round(f / t_fwd / 1e9 / PEAK_BF16_TFLOPS, 4),
                "bwd_ms": round(t_bwd, 4), "bwd_tflops": round(2.5 * f / t_bwd / 1e9, 1),
                "bwd_frac_peak": round(2.5 * f / t_bwd / 1e9 / PEAK_BF16_TFLOPS, 4),
                "causal_fwd_ms": round(t_fwd_c, 4), "causal_bwd_ms": round(t_bwd_c, 4),
                "speedup_vs_causal": round((t_fwd_c + t_bwd_c) / (t_fwd + t_bwd), 3),
                "pairs_ratio": round((n * (n + 1) / 2) / pairs, 3),
            }), flush=True)
        del q, k, v, do, ws, grads
        torch.cuda.empty_cache()


def _decode_line(torch, call, steps, warmup, b, h, nq, nk, d, kv_bytes, splits):
    """One decode JSON line: the per-call time of back-to-back eager calls
    (`eager_ms`, which includes the Python binding's per-call host work when
    that exceeds the GPU time) and of the same calls replayed from a HIP graph
    (`ms`, GPU time); rates from the latter."""
    eager = _time_ms(torch, call, steps, warmup)
    ms = _time_graph_ms(torch, call, steps, warmup)
    gbs = kv_bytes / (ms * 1e-3) / 1e9
    return {"decode": True, "B": b, "H": h, "Nq": nq, "Nk": nk, "d": d, "causal": True, "num_splits": splits,
            "ms": round(ms, 4), "eager_ms": round(eager, 4), "kv_gbs": round(gbs, 1),
            "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}


def decode(torch, E, steps, warmup):
    """Unequal lengths.  Decoding: one query per head after Nk cached tokens
    (B=1, H=32, d=128, causal bottom-right), HBM-bound: reported as the K and V
    bytes read per second against 8 TB/s, with one pass and with the
    library's split-K/V choice; then four query rows (d=128) and one at d=64
    over 16384 keys.  Each decode line gives the eager per-call time and the
    time of the same calls replayed from a HIP graph (rates from the latter).  Chunked prefill: 1024 queries after 7168
    cached tokens (B=1, H=16, d=128, causal): TFLOP/s over the allowed pairs,
    forward (library's split choice) and backward."""
    g = torch.Generator(device="cuda").manual_seed(13)
    b, h, d = 1, 32, 128
    for nk in (4096, 16384, 65536):
        q = torch.randn(b, h, 1, d, device="cuda", generator=g).to(torch.bfloat16)
        k, v = (torch.randn(b, h, nk, d, device="cuda", generator=g).to(torch.bfloat16) for _ in range(2))
        kv_bytes = 2.0 * b * h * nk * d * 2
        o = torch.empty_like(q)
        lse = torch.empty((b, h, 1), dtype=torch.float32, device="cuda")
        for splits in (1, 0):
            nsplit_bytes = E.lib().attn_fwd_qk_workspace_bytes(b, h, 1, nk, d, E.ATTN_BF16, splits)
            ws = torch.empty(max(nsplit_bytes, 256), dtype=torch.uint8, device="cuda")
            call = lambda: E.attn_fwd_qk(q, k, v, causal=True, num_splits=splits, out=o, lse=lse, workspace=ws)
            print(json.dumps(_decode_line(torch, call, steps, warmup, b, h, 1, nk, d, kv_bytes,
                                          "auto" if splits == 0 else splits)), flush=True)
    # The decode kernel's other variants at Nk = 16384: four query rows (as in
    # speculative decoding) and d = 64.
    for nq, dd in ((4, 128), (1, 64)):
        nk = 16384
        q = torch.randn(b, h, nq, dd, device="cuda", generator=g).to(torch.bfloat16)
        k, v = (torch.randn(b, h, nk, dd, device="cuda", generator=g).to(torch.bfloat16) for _ in range(2))
        kv_bytes = 2.0 * b * h * nk * dd * 2
        ws = torch.empty(max(E.lib().attn_fwd_qk_workspace_bytes(b, h, nq, nk, dd, E.ATTN_BF16, 0), 256),
                         dtype=torch.uint8, device="cuda")
        o = torch.empty_like(q)
        lse = torch.empty((b, h, nq), dtype=torch.float32, device="cuda")
        call = lambda: E.attn_fwd_qk(q, k, v, causal=True, num_splits=0, out=o, lse=lse, workspace=ws)
        print(json.dumps(_decode_line(torch, call, steps, warmup, b, h, nq, nk, dd, kv_bytes, "auto")), flush=True)
    b, h, nq, nk = 1, 16, 1024, 8192
    q, do = (torch.randn(b, h, nq, d, device="cuda", generator=g).to(torch.bfloat16) for _ in range(2))
    k, v = (torch.randn(b, h, nk, d, device="cuda", generator=g).to(torch.bfloat16) for _ in range(2))
    pairs = b * h * sum(min(nk, i + (nk - nq) + 1) for i in range(nq))
    o, lse = E.attn_fwd_qk(q, k, v, causal=True, num_splits=0)
    fwd_ms = _time_ms(torch, lambda: E.attn_fwd_qk(q, k, v, causal=True, num_splits=0), steps, warmup)
    bwd_ms = _time_ms(torch, lambda: E.attn_bwd_qk(q, k, v, o, do, lse, causal=True), steps, warmup)
    ff = 4.0 * d * pairs
    print(json.dumps({
        "chunked_prefill": True, "B": b, "H": h, "Nq": nq, "Nk": nk, "d": d, "causal": True,
        "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
        "fwd_tflops": round(ff / fwd_ms / 1e9, 1), "bwd_tflops": round(2.5 * ff / bwd_ms / 1e9, 1),
        "fwd_frac_peak": round(ff / fwd_ms / 1e9 / PEAK_BF16_TFLOPS, 4),
        "bwd_frac_peak": round(2.5 * ff / bwd_ms / 1e9 / PEAK_BF16_TFLOPS, 4),
    }), flush=True)


if __name__ == "__main__":
    main()
