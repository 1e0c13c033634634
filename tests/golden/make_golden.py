"""Write oracle reference values for the large named workloads.

Calls only the float64 oracle (oracle/) on the seeded inputs of
semi_markov_crf_zero_amd/workloads.py and stores compact results as
tests/golden/<name>.npz:

  input_sha256        digest of the four input arrays (the GPU-side test
                      regenerates the inputs and checks this first)
  logz, logz_bwd      [B]
  grad_trans [C,C], grad_dur [K,C]
  rows [B,R]          sampled positions: every multiple of 4096 (the
                      checkpoint boundaries of intervals 4096, 8192, 16384)
                      with its neighbours p-1, p+1 and the burn-in edges
                      p-32, p+32, the first and last valid positions, and
                      random ones
  marginals_rows, grad_rows [B,R,C], boundary_rows [B,R]
                      oracle values at those positions (float32; the bar is
                      1e-4 absolute)
  block [int]         block length of the sums below (4096 positions)
  marginals_blocks, grad_blocks [B,nblock,C], boundary_blocks [B,nblock]
                      sums over every block of positions (float64)
  S_rows [B,R,C], S_last, nu [B,C]  cumulative scores at the sampled rows
  vit_*               Viterbi score, complete segmentation, smallest margin
  path_score [B]      score of the workload's gold path

Usage:  python tests/golden/make_golden.py extreme
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

BLOCK = 4096
R_RANDOM = 128


def input_digest(inp):
    h = hashlib.sha256()
    for k in ("emissions", "lengths", "trans", "dur"):
        h.update(np.ascontiguousarray(inp[k]).tobytes())
    return h.hexdigest()


def sample_rows(lengths, seed=1234):
    rng = np.random.default_rng(seed)
    rows = []
    for L in lengths:
        L = int(L)
        r = [0, L - 1]
        for p in range(BLOCK, L, BLOCK):
            r += [p - 32, p - 1, p, p + 1, p + 32]
        r += list(rng.integers(0, L, size=R_RANDOM))
        rows.append(np.unique(np.clip(np.array(r), 0, L - 1)))
    n = max(len(r) for r in rows)
    # pad with the last row (repeated rows compare the same value twice)
    return np.stack([np.concatenate([r, np.full(n - len(r), r[-1])]) for r in rows]).astype(np.int64)


def block_sums(a, L, T):
    """Sums of a[b, t] over blocks [i*BLOCK, (i+1)*BLOCK) of valid positions."""
    nb = (T + BLOCK - 1) // BLOCK
    out = np.zeros((a.shape[0], nb) + a.shape[2:])
    for b in range(a.shape[0]):
        for i in range(nb):
            lo, hi = i * BLOCK, min((i + 1) * BLOCK, int(L[b]))
            if lo < hi:
                out[b, i] = a[b, lo:hi].sum(axis=0)
    return out


def make(name, nthreads=0):
    t0 = time.time()
    inp = make_inputs(name)
    B, T = inp["B"], inp["T"]
    out = oracle.fwd_bwd(inp, nthreads=nthreads)
    t1 = time.time()
    print("%s: oracle fwd_bwd %.1fs" % (name, t1 - t0), flush=True)
    L = inp["lengths"]
    rows = sample_rows(L)
    bidx = np.arange(B)[:, None]
    res = dict(
        name=np.array(name), input_sha256=np.array(input_digest(inp)),
        logz=out["logz"], logz_bwd=out["logz_bwd"],
        grad_trans=out["grad_trans"], grad_dur=out["grad_dur"],
        rows=rows,
        marginals_rows=out["marginals"][bidx, rows].astype(np.float32),
        grad_rows=out["grad_emissions"][bidx, rows].astype(np.float32),
        boundary_rows=out["boundary"][bidx, rows].astype(np.float32),
        block=np.array(BLOCK),
        marginals_blocks=block_sums(out["marginals"], L, T),
        grad_blocks=block_sums(out["grad_emissions"], L, T),
        boundary_blocks=block_sums(out["boundary"], L, T),
    )
    del out
    nu, S = oracle.prefix(inp)
    res.update(S_rows=S[bidx, rows], S_last=S[np.arange(B), L], nu=nu)
    del S
    vit = oracle.viterbi(inp, nthreads=nthreads)
    print("%s: oracle viterbi %.1fs" % (name, time.time() - t1), flush=True)
    res.update(vit_score=vit["best_score"], vit_num=vit["num_segs"], vit_margin=vit["min_margin"])
    nmax = int(vit["num_segs"].max())
    res["vit_start"] = vit["seg_start"][:, :nmax]
    res["vit_len"] = vit["seg_len"][:, :nmax]
    res["vit_label"] = vit["seg_label"][:, :nmax]
    res["path_score"] = oracle.path_score(inp, inp["gold"])["score"]
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), name + ".npz")
    np.savez_compressed(path, **res)
    print("%s: total %.1fs -> %s" % (name, time.time() - t0, path), flush=True)


if __name__ == "__main__":
    for n in sys.argv[1:] or ["extreme"]:
        make(n)
