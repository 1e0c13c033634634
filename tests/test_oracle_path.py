"""Pin the oracle's path score (oracle/path.py) and boundary posteriors.

The path score is the score of one explicit segmentation; the pins tie it to
quantities fixed independently of its code:
  - explicit enumeration (oracle/bruteforce.py sums every segmentation's
    score from the emissions): equal score for every segmentation, and
    log Z = log sum_y exp(score(y));
  - linearity: central finite differences of the score equal its gradient
    exactly (up to rounding) in x, trans and dur;
  - the identity E_y[grad score(y)] = grad log Z: the probability-weighted
    mean of the path gradients over every segmentation equals the
    enumerated log Z gradients;
  - the Viterbi segmentation scores its own best_score;
  - invalid segmentations (gaps, overlaps, lengths or labels out of range)
    score NaN and contribute nothing.
Boundary posteriors: P(a segment starts at t) is pinned to enumeration in
test_oracle_bruteforce; here its sum over t equals the expected number of
segments, sum_{k,c} of the duration posteriors, and P(start at 0) = 1.
"""
import itertools

import numpy as np
import pytest

from oracle import bruteforce
from oracle.path import path_score
from semi_markov_crf_zero_amd.workloads import make_inputs, make_random, segment_arrays


def _seg_dict(seglists, T):
    B = len(seglists)
    out = {k: np.full((B, T), -1, np.int32) for k in ("seg_start", "seg_len", "seg_label")}
    out["num_segs"] = np.zeros(B, np.int32)
    for b, segs in enumerate(seglists):
        for j, (s, k, c) in enumerate(segs):
            out["seg_start"][b, j], out["seg_len"][b, j], out["seg_label"][b, j] = s, k, c
        out["num_segs"][b] = len(segs)
    return out


@pytest.mark.parametrize("center", [True, False])
@pytest.mark.parametrize("C,K", [(1, 3), (2, 2), (2, 4), (3, 3)])
def test_path_score_matches_enumeration(C, K, center):
    T = 6
    inp = make_random(1, T, C, K, seed=C * 10 + K, tsd=0.5, dsd=0.5)
    items = list(bruteforce.enumerate_sequence(inp["emissions"][0], T, inp["trans"],
                                               inp["dur"], center))
    segs = [it[0] for it in items]
    ref = np.array([it[1] for it in items])
    # score every enumerated segmentation as a batch of one-sequence inputs
    got = []
    for chunk in range(0, len(segs), 64):
        part = segs[chunk:chunk + 64]
        n = len(part)
        batch = dict(emissions=np.repeat(inp["emissions"], n, axis=0),
                     lengths=np.full(n, T, np.int32), trans=inp["trans"], dur=inp["dur"])
        got.append(path_score(batch, _seg_dict(part, T), center=center)["score"])
    got = np.concatenate(got)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    # log Z is the log-sum-exp of the path scores
    bf = bruteforce.brute_force(inp, center=center)
    m = got.max()
    assert abs(m + np.log(np.exp(got - m).sum()) - bf["logz"][0]) < 1e-12


@pytest.mark.parametrize("center", [True, False])
def test_path_gradient_expectation_is_logz_gradient(center):
    """sum_y p(y) grad score(y) = grad log Z (enumeration), every element."""
    C, K, T = 2, 3, 6
    inp = make_random(1, T, C, K, seed=7, tsd=0.4, dsd=0.4)
    items = list(bruteforce.enumerate_sequence(inp["emissions"][0], T, inp["trans"],
                                               inp["dur"], center))
    scores = np.array([sc for _, sc in items])
    p = np.exp(scores - scores.max())
    p /= p.sum()
    acc = {k: 0.0 for k in ("grad_emissions", "grad_trans", "grad_dur")}
    for (segs, _), pi in zip(items, p):
        g = path_score(inp, _seg_dict([segs], T), center=center)
        for k in acc:
            acc[k] = acc[k] + pi * g[k]
    bf = bruteforce.brute_force(inp, center=center)
    for k in acc:
        np.testing.assert_allclose(acc[k], bf[k], rtol=0, atol=1e-12, err_msg=k)


def test_path_gradient_finite_differences():
    """The score is linear in x, trans and dur: central differences equal the
    gradient up to rounding, for every element (weights included)."""
    inp = make_inputs("tiny")
    T = inp["T"]
    gold = inp["gold"]
    w = np.array([1.0, -0.5, 2.0, 0.25])
    g = path_score(inp, gold, weights=w)
    base = {k: np.asarray(inp[k], np.float64) for k in ("emissions", "trans", "dur")}
    h = 0.5
    rng = np.random.default_rng(3)
    for key, gk in (("emissions", "grad_emissions"), ("trans", "grad_trans"), ("dur", "grad_dur")):
        idx = [tuple(rng.integers(0, n) for n in base[key].shape) for _ in range(40)]
        for ix in idx:
            vals = []
            for sgn in (1, -1):
                arr = base[key].copy()
                arr[ix] += sgn * h
                mod = dict(inp)
                mod[key] = arr
                vals.append(float(np.dot(w, path_score(mod, gold)["score"])))
            fd = (vals[0] - vals[1]) / (2 * h)
            assert abs(fd - g[gk][ix]) < 1e-9, (key, ix, fd, g[gk][ix])
    assert T == 256


def test_viterbi_path_scores_its_best_score(oracle_mod):
    for name in ("tiny", "nlp"):
        inp = make_inputs(name)
        v = oracle_mod.viterbi(inp)
        ps = path_score(inp, v)["score"]
        np.testing.assert_allclose(ps, v["best_score"], rtol=1e-12, atol=1e-9)


def test_invalid_segmentations_score_nan():
    inp = make_random(6, 8, 3, 4, seed=1)
    T = 8
    bad = [
        [(0, 4, 0), (4, 3, 1)],              # ends short of L
        [(0, 4, 0), (3, 5, 1)],              # overlap
        [(0, 5, 0), (5, 3, 1)],              # length 5 > K = 4
        [(0, 4, 3), (4, 4, 1)],              # label 3 >= C
        [(1, 4, 0), (5, 3, 1)],              # does not start at 0
        [(0, 4, 0), (4, 4, 2)],              # valid
    ]
    out = path_score(inp, _seg_dict(bad, T))
    assert np.all(np.isnan(out["score"][:5])) and np.isfinite(out["score"][5])
    assert np.all(out["grad_emissions"][:5] == 0)
    assert out["grad_trans"].sum() == 1 and out["grad_dur"].sum() == 2


def test_boundary_sums_to_expected_segment_count(oracle_mod):
    for name in ("tiny", "nlp"):
        inp = make_inputs(name)
        o = oracle_mod.fwd_bwd(inp)
        L = inp["lengths"]
        assert np.allclose(o["boundary"][:, 0], 1.0, atol=1e-12)
        for b in range(inp["B"]):
            assert np.all(o["boundary"][b, L[b]:] == 0)
            assert np.all(o["boundary"][b] >= -1e-15) and np.all(o["boundary"][b] <= 1 + 1e-12)
        # sum_t P(start at t) = E[#segments] = sum_{k,c} P(duration k, label c)
        np.testing.assert_allclose(o["boundary"].sum(), o["grad_dur"].sum(), rtol=1e-10)


def test_segment_arrays_tile_each_length():
    for name in ("tiny", "nlp", "speech"):
        inp = make_inputs(name)
        g = inp["gold"]
        for b in range(inp["B"]):
            n = g["num_segs"][b]
            assert g["seg_start"][b, 0] == 0
            ends = g["seg_start"][b, :n] + g["seg_len"][b, :n]
            assert ends[-1] == inp["lengths"][b]
            assert np.all(g["seg_start"][b, 1:n] == ends[:-1])
            assert np.all((g["seg_len"][b, :n] >= 1) & (g["seg_len"][b, :n] <= inp["K"]))
            assert np.all(g["seg_start"][b, n:] == -1)
    assert segment_arrays([], [], 4)["num_segs"].shape == (0,)
