"""Closed forms of the semi-CRF partition function for zero potentials.

TEST INFRASTRUCTURE ONLY.  With x = 0, trans = 0 and dur = 0 every labelled
segmentation scores 0, so Z(L) is the number of labelled segmentations of
[0, L) into segments of length 1..K with C labels each.  Splitting off the
last segment gives the integer recursion

    z[0] = 1,   z[t] = C * sum_{k=1}^{min(K,t)} z[t-k]

and for K >= L the count is C * (C + 1)^(L - 1) (each of the L - 1 gaps is
either not a boundary or a boundary followed by one of C labels).  Counting
argument only; no dynamic programme of the library or of the oracle is used.
"""
from __future__ import annotations

import math


def log_count(L, C, K):
    """log z[L] computed with exact Python integers."""
    z = [1]
    for t in range(1, L + 1):
        z.append(C * sum(z[t - k] for k in range(1, min(K, t) + 1)))
    n = z[L]
    # log of a big integer without overflow
    bits = n.bit_length()
    if bits < 1000:
        return math.log(n)
    shift = bits - 60
    return math.log(n >> shift) + shift * math.log(2.0)


def log_count_unbounded(L, C):
    """K >= L: log(C (C+1)^(L-1))."""
    return math.log(C) + (L - 1) * math.log(C + 1)


def log_count_float(L, C, K):
    """Same recursion evaluated in log space with a sliding window (any L)."""
    logs = [0.0]
    for t in range(1, L + 1):
        terms = [logs[t - k] for k in range(1, min(K, t) + 1)]
        m = max(terms)
        logs.append(math.log(C) + m + math.log(sum(math.exp(a - m) for a in terms)))
    return logs[L]
