"""Expected decode outputs of the two largest workloads, computed by the oracle
alone (oracle.decode_reference) from the seeded inputs: every request of the long
workload at every decode step, every request of the prefix workload at four
steps (the first, two inside and the last), and every request of the prefix
workload with FP8 KV storage (reading R20) at the first and the last step.

    python tests/golden/make_fullsize.py [--procs 8] [--only prefix|long|prefix_fp8kv]

writes tests/golden/prefix_decode.npz, tests/golden/long_decode.npz and
tests/golden/prefix_decode_fp8kv.npz:
  req [n], step [n], L [n]   request, decode step (0-based), length after the append
  idx [n][k] int32           top-k ordinals (ascending, -1 padded)
  out [n][16][128] float32   attention output (computed in float64)
Nothing here comes from the GPU path; tests/test_gpu_fullsize.py compares the GPU
against these files.
"""

from __future__ import annotations

import argparse
import multiprocessing as mp
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import decode_reference  # noqa: E402
from synth.workloads import RequestTokens, make  # noqa: E402

# (workload index, file, requests (None: all), decode steps, KV storage)
SAMPLES = {
    "prefix": (3, "prefix_decode.npz", None, (0, 10, 21, 31), "bf16"),
    "long": (5, "long_decode.npz", None, tuple(range(16)), "bf16"),
    "prefix_fp8kv": (3, "prefix_decode_fp8kv.npz", None, (0, 31), "fp8"),
}


def run(name: str, procs: int) -> None:
    index, fname, reqs, steps, kv = SAMPLES[name]
    wl = make(index)
    if reqs is None:
        reqs = list(range(wl.batch))
    Wc, Wh = synth.gate_weights(wl.seed)
    rows = {"req": [], "step": [], "L": [], "idx": [], "out": []}
    with mp.get_context("fork").Pool(procs) as pool:
        for b in reqs:
            t0 = time.time()
            src = RequestTokens(index, b)
            cases = []
            for t in steps:
                p = int(wl.prefill[b]) + t          # position of the step's new token
                q, qi = src.query(p)
                cases.append((p + 1, q, qi, wl.topk))
            res = decode_reference(src, wl.n_win, Wc, Wh, cases, pmap=pool.map, chunk=16, kv_format=kv)
            for t, (L, *_), (idx, _, out) in zip(steps, cases, res):
                rows["req"].append(b)
                rows["step"].append(t)
                rows["L"].append(L)
                rows["idx"].append(idx.astype(np.int32))
                rows["out"].append(out.astype(np.float32))
            print(f"{name}: request {b} (L0 {int(wl.prefill[b])}) done in {time.time() - t0:.0f} s",
                  flush=True)
    np.savez_compressed(os.path.join(HERE, fname), req=np.array(rows["req"], np.int32),
                        step=np.array(rows["step"], np.int32), L=np.array(rows["L"], np.int64),
                        idx=np.stack(rows["idx"]), out=np.stack(rows["out"]))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--procs", type=int, default=8)
    ap.add_argument("--only", choices=sorted(SAMPLES), default=None)
    a = ap.parse_args()
    for name in ([a.only] if a.only else sorted(SAMPLES, key=lambda n: n != "prefix")):
        run(name, a.procs)


if __name__ == "__main__":
    main()
