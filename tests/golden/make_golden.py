"""Write oracle reference values for the large named workloads.

Calls only the float64 oracle (oracle/) on the seeded inputs of
semi_markov_crf_zero_amd/workloads.py and stores compact results as
tests/golden/<name>.npz:

  input_sha256        digest of the four input arrays (the GPU-side test
                      regenerates the inputs and checks this first)
  logz, logz_bwd      [B]
  grad_trans [C,C], grad_dur [K,C]
  rows [B,R]          sampled positions (first, last valid, and random ones)
  marginals_rows, grad_rows [B,R,C]   oracle values at those positions (stored
                                      as float32; the tolerance is 1e-4 absolute)
  S_rows [B,R/4,C], S_last, nu [B,C]  cumulative scores at every 4th sampled row
  colsum_marginals [B,C]              sum_i mu[b,i,c]
  vit_*                               Viterbi score, segments, smallest margin

Usage:  python tests/golden/make_golden.py speech genome extreme
"""
from __future__ import annotations

import hashlib
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from semi_markov_crf_zero_amd.workloads import make_inputs  # noqa: E402

R_MAX = 254


def n_random_rows(C):
    # keep each fixture small: about 8K sampled values per sequence
    return max(16, min(R_MAX, 8192 // C))


def input_digest(inp):
    h = hashlib.sha256()
    for k in ("emissions", "lengths", "trans", "dur"):
        h.update(np.ascontiguousarray(inp[k]).tobytes())
    return h.hexdigest()


def sample_rows(lengths, C, seed=1234):
    rng = np.random.default_rng(seed)
    R = n_random_rows(C)
    rows = []
    for L in lengths:
        L = int(L)
        r = np.unique(np.concatenate([[0, L - 1], rng.integers(0, L, size=R)]))
        while r.size < min(R + 2, L):
            r = np.unique(np.concatenate([r, rng.integers(0, L, size=R + 2 - r.size)]))
        rows.append(np.sort(r)[:R + 2])
    return np.stack(rows).astype(np.int64)


def make(name, nthreads=0):
    t0 = time.time()
    inp = make_inputs(name)
    B, T, C, K = inp["B"], inp["T"], inp["C"], inp["K"]
    out = oracle.fwd_bwd(inp, nthreads=nthreads)
    t1 = time.time()
    vit = oracle.viterbi(inp, nthreads=nthreads)
    nu, S = oracle.prefix(inp)
    rows = sample_rows(inp["lengths"], C)
    bidx = np.arange(B)[:, None]
    res = dict(
        name=np.array(name), input_sha256=np.array(input_digest(inp)),
        logz=out["logz"], logz_bwd=out["logz_bwd"],
        grad_trans=out["grad_trans"], grad_dur=out["grad_dur"],
        rows=rows,
        marginals_rows=out["marginals"][bidx, rows].astype(np.float32),
        grad_rows=out["grad_emissions"][bidx, rows].astype(np.float32),
        S_rows=S[bidx, rows[:, ::4]], S_last=S[np.arange(B), inp["lengths"]], nu=nu,
        colsum_marginals=out["marginals"].sum(axis=1),
        vit_score=vit["best_score"], vit_num=vit["num_segs"], vit_margin=vit["min_margin"],
    )
    nmax = int(vit["num_segs"].max())
    res["vit_start"] = vit["seg_start"][:, :nmax]
    res["vit_len"] = vit["seg_len"][:, :nmax]
    res["vit_label"] = vit["seg_label"][:, :nmax]
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), name + ".npz")
    np.savez_compressed(path, **res)
    print("%s: oracle fwd_bwd %.1fs, total %.1fs -> %s" % (name, t1 - t0, time.time() - t0, path),
          flush=True)


if __name__ == "__main__":
    for n in sys.argv[1:] or ["speech", "genome", "extreme"]:
        make(n)
