"""Seeded synthetic semi-CRF inputs.

This module only draws random numbers: it contains none of the semi-CRF
arithmetic, so both the float64 oracle (tests) and the HIP path (tests,
bench) can consume the same arrays without sharing any method code.

Every array is drawn in float64 from ``numpy.random.default_rng(seed)``
(PCG64) and cast once to float32; both sides consume the cast values.
Normal distributions are written N(0, s) with ``s`` the standard deviation.

Draw order, per config: lengths -> per-sequence path segment lengths ->
path labels -> emission noise -> trans -> dur.  Positions t >= lengths[b]
are drawn like the others and must be ignored by every consumer.

The five named workloads follow the shapes of the pages' NLP-, speech- and
genome-scale settings ("Streaming Structured Inference with Flash-SemiCRF",
abstract and the technical summary's results section); no public dataset is
used or reproduced.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    C: int
    K: int
    description: str


WORKLOADS = {
    "tiny": Workload("tiny", 4, 256, 8, 16,
                     "B=4 T=256 C=8 K=16; lengths=T; x~N(0,1); trans,dur~N(0,0.1)"),
    "nlp": Workload("nlp", 32, 512, 24, 32,
                    "B=32 T=512 C=24 K=32; lengths~U[T/2,T]; x~N(0,1)+2.0 on a gold path "
                    "(segment lengths U{1..K}); trans,dur~N(0,0.1)"),
    "speech": Workload("speech", 16, 4096, 256, 64,
                       "B=16 T=4096 C=256 K=64; lengths=T; x~N(0,1)+1.5 on a path with lengths "
                       "min(Geom(1/12),K); trans~N(0,0.05); dur=-0.05k+N(0,0.1)"),
    "genome": Workload("genome", 4, 131072, 16, 512,
                       "B=4 T=131072 C=16 K=512; lengths=T; path lengths U{50..K}, label 0 w.p. 0.7 "
                       "else U{1..15}; x~N(0,1)+1.0 on the path; trans,dur~N(0,0.1)"),
    "extreme": Workload("extreme", 1, 1048576, 64, 256,
                        "B=1 T=1048576 C=64 K=256; lengths=T; x~N(0,1)+1.0 on a path with lengths "
                        "U{1..K}; trans,dur~N(0,0.1)"),
}


def _path(rng, T, K, C, kind):
    """Draw one labelled segment path over [0, T) (truncated at T).

    Returns (seg_lengths, seg_labels) as int arrays, segment lengths drawn
    first, labels second (the fixed draw order)."""
    if kind == "uniform1K":
        lens = rng.integers(1, K + 1, size=T)
    elif kind == "geom12":
        lens = np.minimum(rng.geometric(1.0 / 12.0, size=T), K)
    elif kind == "genome":
        lens = rng.integers(50, K + 1, size=T // 50 + 2)
    else:
        raise ValueError(kind)
    ends = np.cumsum(lens)
    n = int(np.searchsorted(ends, T) + 1)
    lens = lens[:n].copy()
    lens[-1] -= int(ends[n - 1] - T)
    if kind == "genome":
        is_zero = rng.random(n) < 0.7
        other = rng.integers(1, C, size=n)
        labels = np.where(is_zero, 0, other)
    else:
        labels = rng.integers(0, C, size=n)
    return lens.astype(np.int64), labels.astype(np.int64)


def segment_arrays(paths, lengths, T):
    """Segment lists in the layout of the library's segmentation arguments:
    seg_start / seg_len / seg_label [B,T] int32 (-1 past num_segs) and
    num_segs [B], each path cut at its sequence's length."""
    B = len(paths)
    out = {k: np.full((B, T), -1, dtype=np.int32) for k in ("seg_start", "seg_len", "seg_label")}
    out["num_segs"] = np.zeros(B, dtype=np.int32)
    for b, (lens, labels) in enumerate(paths):
        L = int(lengths[b])
        pos = 0
        j = 0
        for k, c in zip(lens, labels):
            if pos >= L:
                break
            k = min(int(k), L - pos)
            out["seg_start"][b, j] = pos
            out["seg_len"][b, j] = k
            out["seg_label"][b, j] = int(c)
            pos += k
            j += 1
        out["num_segs"][b] = j
    return out


def _paint(x_b, lens, labels, amount):
    pos = 0
    for L, c in zip(lens, labels):
        x_b[pos:pos + L, c] += amount
        pos += L


def make_inputs(name: str, seed: int = 0):
    """Return a dict with emissions [B,T,C] f32, lengths [B] i32,
    trans [C,C] f32, dur [K,C] f32, the shape ints for a named workload and
    `gold`, the path the emissions were raised on (segment arrays of
    segment_arrays(), cut at each length; for tiny, whose emissions have no
    path, one drawn afterwards from a separate generator)."""
    w = WORKLOADS[name]
    B, T, C, K = w.B, w.T, w.C, w.K
    rng = np.random.default_rng(seed)
    if name == "nlp":
        lengths = rng.integers(T // 2, T + 1, size=B)
    else:
        lengths = np.full(B, T)
    paths = []
    if name != "tiny":
        kind = {"nlp": "uniform1K", "speech": "geom12", "genome": "genome",
                "extreme": "uniform1K"}[name]
        paths = [_path(rng, T, K, C, kind) for _ in range(B)]
    x = rng.standard_normal((B, T, C))
    if name != "tiny":
        amount = {"nlp": 2.0, "speech": 1.5, "genome": 1.0, "extreme": 1.0}[name]
        for b in range(B):
            _paint(x[b], paths[b][0], paths[b][1], amount)
    tsd = 0.05 if name == "speech" else 0.1
    trans = rng.normal(0.0, tsd, size=(C, C))
    dur = rng.normal(0.0, 0.1, size=(K, C))
    if name == "speech":
        dur = dur - 0.05 * np.arange(1, K + 1)[:, None]
    if name == "tiny":
        rng2 = np.random.default_rng(seed + 1)
        paths = [_path(rng2, T, K, C, "uniform1K") for _ in range(B)]
    return dict(
        B=B, T=T, C=C, K=K,
        gold=segment_arrays(paths, lengths, T),
        emissions=np.ascontiguousarray(x, dtype=np.float32),
        lengths=np.ascontiguousarray(lengths, dtype=np.int32),
        trans=np.ascontiguousarray(trans, dtype=np.float32),
        dur=np.ascontiguousarray(dur, dtype=np.float32),
    )


def make_random(B, T, C, K, seed=0, sigma=1.0, tsd=0.1, dsd=0.1, lengths=None,
                pad_value=None):
    """Generic iid inputs for parity grids and edge cases.

    ``lengths`` may be given explicitly (list/array); otherwise all equal T.
    ``pad_value`` (e.g. NaN) overwrites every position t >= lengths[b]."""
    rng = np.random.default_rng(seed)
    if lengths is None:
        lengths = np.full(B, T)
    lengths = np.asarray(lengths, dtype=np.int32)
    x = rng.normal(0.0, sigma, size=(B, T, C))
    trans = rng.normal(0.0, tsd, size=(C, C))
    dur = rng.normal(0.0, dsd, size=(K, C))
    x = x.astype(np.float32)
    if pad_value is not None:
        for b in range(B):
            x[b, int(lengths[b]):, :] = pad_value
    return dict(B=B, T=T, C=C, K=K,
                emissions=np.ascontiguousarray(x),
                lengths=np.ascontiguousarray(lengths),
                trans=np.ascontiguousarray(trans, dtype=np.float32),
                dur=np.ascontiguousarray(dur, dtype=np.float32))
