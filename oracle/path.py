"""Score of a given labelled segmentation and its gradients, from the
definition (float64, plain numpy).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The training loss of a semi-CRF is log Z - score(gold) ("Streaming
Structured Inference with Flash-SemiCRF", technical summary at gist.science,
section 3: training on labelled segmentations).  The score of a segmentation
(s_j, k_j, c_j) of [0, L) is summed straight from the emissions, as in the
definition of the model (abstract: segment content from cumulative sums of
baseline-subtracted emissions; technical summary, section 2.C: the baseline
nu is the per-label mean over the sequence):

  score = sum_j [ sum_{i in [s_j, s_j + k_j)} (x[i, c_j] - nu[c_j]) + dur[k_j - 1, c_j] ]
        + sum_{j >= 1} trans[c_{j-1}, c_j]

It is linear in x, trans and dur, so its gradient is a count:
  d score / d x[i, c]        = 1[position i has label c] - (1/L) #(positions of label c)
                               (the second term only with centring, through nu)
  d score / d trans[c', c]   = #(j >= 1 with c_{j-1} = c', c_j = c)
  d score / d dur[k - 1, c]  = #(segments of length k and label c)
For a batch, F = sum_b w_b score_b; an invalid segmentation (not a tiling of
[0, L) by segments of length 1..K with labels in [0, C)) scores NaN and
contributes nothing.
"""
from __future__ import annotations

import numpy as np


def segments_of(seg, b):
    """List of (start, length, label) of sequence b from the [B,T] arrays."""
    n = int(seg["num_segs"][b])
    return [(int(seg["seg_start"][b, j]), int(seg["seg_len"][b, j]), int(seg["seg_label"][b, j]))
            for j in range(n)]


def is_valid(segs, L, C, K):
    if not segs or len(segs) > L:
        return False
    pos = 0
    for (s, k, c) in segs:
        if s != pos or not (1 <= k <= K) or not (0 <= c < C):
            return False
        pos += k
    return pos == L


def path_score(inp, seg, center=True, weights=None):
    """Returns dict(score [B], grad_emissions [B,T,C], grad_trans [C,C],
    grad_dur [K,C]) in float64 for the segmentations `seg` (dict of
    seg_start, seg_len, seg_label [B,T] and num_segs [B])."""
    x = np.asarray(inp["emissions"], dtype=np.float64)
    lengths = np.asarray(inp["lengths"])
    trans = np.asarray(inp["trans"], dtype=np.float64)
    dur = np.asarray(inp["dur"], dtype=np.float64)
    B, T, C = x.shape
    K = dur.shape[0]
    w = np.ones(B) if weights is None else np.asarray(weights, dtype=np.float64)
    score = np.full(B, np.nan)
    gx = np.zeros((B, T, C))
    gt = np.zeros((C, C))
    gd = np.zeros((K, C))
    for b in range(B):
        L = int(lengths[b])
        segs = segments_of(seg, b)
        if not (1 <= L <= T) or not is_valid(segs, L, C, K):
            continue
        xb = x[b, :L]
        nu = xb.mean(axis=0) if center else np.zeros(C)
        sc = 0.0
        count = np.zeros(C)
        prev = None
        for (s, k, c) in segs:
            sc += float(np.sum(xb[s:s + k, c] - nu[c])) + float(dur[k - 1, c])
            gx[b, s:s + k, c] += w[b]
            count[c] += k
            gd[k - 1, c] += w[b]
            if prev is not None:
                sc += float(trans[prev, c])
                gt[prev, c] += w[b]
            prev = c
        if center:
            gx[b, :L] -= w[b] * count[None, :] / L
        score[b] = sc
    return dict(score=score, grad_emissions=gx, grad_trans=gt, grad_dur=gd)
