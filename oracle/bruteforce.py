"""Explicit enumeration of every labelled segmentation (tiny inputs only).

TEST INFRASTRUCTURE ONLY.  This is the semi-CRF written as its definition
(abstract of "Streaming Structured Inference with Flash-SemiCRF": a
distribution over segmentations into labelled segments, exact inference;
technical summary section 2.A/2.C: segment content score from cumulative
sums of baseline-subtracted emissions):

  score(y) = sum_j [ sum_{i in seg j} (x[i,c_j] - nu[c_j]) + dur[k_j - 1, c_j] ]
             + sum_{j>=2} trans[c_{j-1}, c_j]

summed directly from the emissions (no prefix-sum array, no recursion), and
every expectation is an explicit probability-weighted sum over all y.
Feasible for L <= 8, C <= 3 (at most 128 compositions x 3^8 labellings).
"""
from __future__ import annotations

import itertools

import numpy as np


def compositions(L, K):
    """All ordered tuples of segment lengths in [1, K] summing to L."""
    out = []

    def rec(rem, acc):
        if rem == 0:
            out.append(tuple(acc))
            return
        for k in range(1, min(K, rem) + 1):
            acc.append(k)
            rec(rem - k, acc)
            acc.pop()

    rec(L, [])
    return out


def enumerate_sequence(x, L, trans, dur, center=True):
    """Yield (segments, score) for every labelled segmentation of [0, L).

    x: [T, C] float64 (rows >= L ignored); segments: list of (start, k, c)."""
    x = np.asarray(x, dtype=np.float64)[:L]
    C = x.shape[1]
    K = dur.shape[0]
    nu = x.mean(axis=0) if center else np.zeros(C)
    for comp in compositions(L, K):
        starts = np.concatenate([[0], np.cumsum(comp)[:-1]]).astype(int)
        for labels in itertools.product(range(C), repeat=len(comp)):
            score = 0.0
            segs = []
            for j, (s, k, c) in enumerate(zip(starts, comp, labels)):
                score += float(np.sum(x[s:s + k, c] - nu[c])) + float(dur[k - 1, c])
                if j > 0:
                    score += float(trans[labels[j - 1], c])
                segs.append((int(s), int(k), int(c)))
            yield segs, score


def _lse(a):
    a = np.asarray(a, dtype=np.float64)
    m = a.max()
    return float(m + np.log(np.sum(np.exp(a - m))))


def brute_force(inp, center=True, grad_logz=None):
    """Exact log Z, coverage marginals, parameter gradients and the MAP
    segmentation by enumeration.  Returns a dict like oracle.fwd_bwd plus
    'viterbi' = list of (best_score, segments) per sequence, where among
    maximisers the first in enumeration order is kept; 'viterbi_ties' lists
    every segmentation within rounding (1e-9 relative) of the maximum;
    'boundary' [B,T] is the probability that a segment starts at t."""
    x = np.asarray(inp["emissions"], dtype=np.float64)
    lengths = np.asarray(inp["lengths"])
    trans = np.asarray(inp["trans"], dtype=np.float64)
    dur = np.asarray(inp["dur"], dtype=np.float64)
    B, T, C = x.shape
    K = dur.shape[0]
    w = np.ones(B) if grad_logz is None else np.asarray(grad_logz, dtype=np.float64)
    logz = np.zeros(B)
    mu = np.zeros((B, T, C))
    gx = np.zeros((B, T, C))
    gt = np.zeros((C, C))
    gd = np.zeros((K, C))
    bnd = np.zeros((B, T))
    vit = []
    ties = []
    for b in range(B):
        L = int(lengths[b])
        items = list(enumerate_sequence(x[b], L, trans, dur, center))
        scores = np.array([sc for _, sc in items])
        lz = _lse(scores)
        logz[b] = lz
        probs = np.exp(scores - lz)
        for (segs, _), p in zip(items, probs):
            prev = None
            for (s, k, c) in segs:
                mu[b, s:s + k, c] += p
                bnd[b, s] += p
                gd[k - 1, c] += w[b] * p
                if prev is not None:
                    gt[prev, c] += w[b] * p
                prev = c
        if center:
            gx[b, :L] = w[b] * (mu[b, :L] - mu[b, :L].mean(axis=0, keepdims=True))
        else:
            gx[b, :L] = w[b] * mu[b, :L]
        best = scores.max()
        # maximisers up to rounding: reordering segment lengths inside a run of
        # one label gives exactly equal scores in real arithmetic
        idx = [i for i in range(len(items)) if scores[i] >= best - 1e-9 * (abs(best) + 1.0)]
        vit.append((float(best), items[idx[0]][0]))
        ties.append([items[i][0] for i in idx])
    return dict(logz=logz, marginals=mu, grad_emissions=gx, grad_trans=gt, grad_dur=gd,
                boundary=bnd, viterbi=vit, viterbi_ties=ties)


def path_score(x, L, trans, dur, segs, center=True):
    """Score of one explicit segmentation, summed from the emissions."""
    x = np.asarray(x, dtype=np.float64)[:L]
    nu = x.mean(axis=0) if center else np.zeros(x.shape[1])
    score = 0.0
    prev = None
    for (s, k, c) in segs:
        score += float(np.sum(x[s:s + k, c] - nu[c])) + float(dur[k - 1, c])
        if prev is not None:
            score += float(trans[prev, c])
        prev = c
    return score
