"""Textbook linear-chain CRF, the K=1 special case of the semi-CRF.

TEST INFRASTRUCTURE ONLY.  The technical summary of "Streaming Structured
Inference with Flash-SemiCRF" (section 1) names the linear-chain CRF as the
K=1 restriction of the model.  With K=1 every segment has length one, so a
labelling y of [0, L) scores

    sum_i (x[i, y_i] - nu[y_i] + dur[0, y_i]) + sum_{i>=1} trans[y_{i-1}, y_i]

This module evaluates that model independently of the semi-CRF code: log Z
as a product of C x C matrices in probability space (rescaled every step),
and the MAP labelling with the classic per-position Viterbi over labels.
"""
from __future__ import annotations

import numpy as np


def unaries(x, L, dur, center=True):
    x = np.asarray(x, dtype=np.float64)[:L]
    nu = x.mean(axis=0) if center else np.zeros(x.shape[1])
    return x - nu[None, :] + np.asarray(dur, dtype=np.float64)[0][None, :]


def log_partition(x, L, trans, dur, center=True):
    """log Z = log( 1^T diag(e_0) prod_{i>=1} (exp(trans) diag(e_i)) 1 ),
    evaluated left to right with a running log scale."""
    un = unaries(x, L, dur, center)
    E = np.exp(np.asarray(trans, dtype=np.float64))
    vec = np.exp(un[0] - un[0].max())
    logscale = un[0].max()
    for i in range(1, L):
        m = un[i].max()
        vec = (vec @ E) * np.exp(un[i] - m)
        logscale += m
        s = vec.sum()
        vec /= s
        logscale += np.log(s)
    return float(logscale + np.log(vec.sum()))


def viterbi(x, L, trans, dur, center=True):
    """MAP labelling; ties go to the smallest previous label and, at the end,
    to the smallest final label.  Returns (score, labels)."""
    un = unaries(x, L, dur, center)
    tr = np.asarray(trans, dtype=np.float64)
    C = un.shape[1]
    delta = un[0].copy()
    back = np.zeros((L, C), dtype=int)
    for i in range(1, L):
        cand = delta[:, None] + tr  # [prev, cur]
        back[i] = np.argmax(cand, axis=0)  # first maximum = smallest prev label
        delta = cand[back[i], np.arange(C)] + un[i]
    last = int(np.argmax(delta))
    labels = [last]
    for i in range(L - 1, 0, -1):
        labels.append(int(back[i, labels[-1]]))
    return float(delta[last]), labels[::-1]
