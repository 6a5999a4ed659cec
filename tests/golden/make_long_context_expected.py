"""Write the float64 oracle's dK and dV for sampled key rows of the long-context workload.

Workload: B=1, H=8, N=65536, d=64, bf16 inputs drawn by ``synth.qkvdo`` with the
workload's seed, causal, scale 1/sqrt(d).  The key-row gradients dK_j and dV_j
need the softmax statistics (LSE_i and D_i) of every query row of the head, a
full N x N pass per head, so they are computed once here, with the oracle only,
and stored in ``long_n65536_d64_causal_key_rows.npz`` next to this script.
Query-row values (O, LSE, dQ) are cheap and are computed by the test itself.

Usage: ``python tests/golden/make_long_context_expected.py`` (about a minute on
8 cores; heads run in parallel processes).
"""

import hashlib
import os
import sys
from concurrent.futures import ProcessPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
os.environ.setdefault("OPENBLAS_NUM_THREADS", "1")

import numpy as np  # noqa: E402

import synth  # noqa: E402
from oracle import attention as A  # noqa: E402

NAME = "long_n65536_d64_causal"
OUT = os.path.join(HERE, NAME + "_key_rows.npz")
KEY_SAMPLE_SEED_OFFSET = 2  # key pairs use seed + 2; query pairs use seed + 1
COUNT = 512


def fingerprint(inp):
    h = hashlib.sha256()
    for name in ("q", "k", "v", "do"):
        h.update(np.ascontiguousarray(inp[name + "_raw"]).tobytes())
    return h.hexdigest()


def _head_job(args):
    hd, cols = args
    w = synth.WORKLOADS[NAME]
    inp = synth.qkvdo(w.seed, w.shape, w.dtype)
    q, k, v, do = (inp[x].reshape(w.b * w.h, w.n, w.d)[hd] for x in ("q", "k", "v", "do"))
    scale = 1.0 / np.sqrt(w.d)
    lse, dsum = A.head_row_stats(q, k, v, do, w.causal, scale, chunk=1024)
    dk, dv = A.backward_key_rows(q, k, v, do, cols, lse, dsum, w.causal, scale)
    return hd, dk, dv


def main():
    w = synth.WORKLOADS[NAME]
    pairs = synth.sample_pairs(w.seed + KEY_SAMPLE_SEED_OFFSET, w.b * w.h, w.n, COUNT)
    inp = synth.qkvdo(w.seed, w.shape, w.dtype)
    fp = fingerprint(inp)
    del inp
    heads = np.unique(pairs[:, 0])
    jobs = [(int(hd), pairs[pairs[:, 0] == hd, 1]) for hd in heads]
    dk = np.zeros((COUNT, w.d))
    dv = np.zeros((COUNT, w.d))
    with ProcessPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for hd, dk_h, dv_h in ex.map(_head_job, jobs):
            sel = pairs[:, 0] == hd
            dk[sel] = dk_h
            dv[sel] = dv_h
            print("head", hd, "done", flush=True)
    np.savez_compressed(OUT, pairs=pairs, dk=dk, dv=dv, inputs_sha256=np.array(fp))
    print("wrote", OUT)


if __name__ == "__main__":
    main()
