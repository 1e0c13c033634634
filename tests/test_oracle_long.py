"""Pins of the float64 oracle at long sequence lengths (genome and extreme
scale), where the enumeration pins cannot reach.

* Zero potentials at T = 2^20, K = 2: every labelled segmentation scores 0,
  so Z is their number.  For K = 2 the count obeys z[t] = C (z[t-1] + z[t-2])
  (z[0] = 1, z[1] = C), a linear recurrence with the closed form
  z[t] = A r1^t + B r2^t, r1,2 = (C +- sqrt(C^2 + 4C)) / 2: log Z at any
  length without a loop.  By the symmetry of the labels every marginal is
  1/C, the emission gradients vanish (centred), and the parameter gradients
  obey the counting identities.
* Time reversal at T = 2^17: reversing the emissions and transposing the
  transitions maps every segmentation to its mirror image with the same
  score, so log Z is unchanged and every output mirrors (marginals and
  emission gradients reversed in t, grad_trans transposed, grad_dur equal,
  P(segment starts at t) = P(segment ends at L - t)).  The oracle computes the
  two problems along different paths (its forward table of one is the
  backward table of the other), so an index or sign slip in either breaks
  the symmetry.
"""
import math

import numpy as np

from semi_markov_crf_zero_amd.workloads import make_random


def _closed_form_k2(L, C):
    d = math.sqrt(C * C + 4.0 * C)
    r1, r2 = (C + d) / 2.0, (C - d) / 2.0
    a = (C - r2) / (r1 - r2)
    b = 1.0 - a
    # log z[L] = log a + L log r1 + log(1 + (b/a) (r2/r1)^L); |r2/r1| < 1
    return math.log(a) + L * math.log(r1) + math.log1p((b / a) * (r2 / r1) ** L)


def test_zero_potentials_closed_form_at_2_20(oracle_mod):
    C, K, L = 3, 2, 1 << 20
    # the closed form agrees with the integer recursion where both are cheap
    from oracle import closed_form
    for n in (1, 2, 3, 10, 300):
        assert abs(_closed_form_k2(n, C) - closed_form.log_count(n, C, K)) < 1e-12 * max(1, n)
    inp = dict(emissions=np.zeros((1, L, C), np.float32), lengths=np.array([L], np.int32),
               trans=np.zeros((C, C), np.float32), dur=np.zeros((K, C), np.float32))
    # one thread: at C = 3 a position is a few dozen operations, far less than
    # the thread synchronisation the oracle's per-position parallel loops cost
    o = oracle_mod.fwd_bwd(inp, nthreads=1)
    ref = _closed_form_k2(L, C)
    assert abs(o["logz"][0] - ref) <= 1e-12 * abs(ref), (o["logz"][0], ref)
    assert abs(o["logz_bwd"][0] - ref) <= 1e-12 * abs(ref)
    assert np.abs(o["marginals"][0] - 1.0 / C).max() < 1e-10
    assert np.abs(o["grad_emissions"][0]).max() < 1e-10
    # sum_k k grad_dur = L; transitions = segments - 1; labels symmetric
    gd, gt = o["grad_dur"], o["grad_trans"]
    assert abs((np.arange(1, K + 1)[:, None] * gd).sum() - L) < 1e-6 * L
    assert abs(gt.sum() - (gd.sum() - 1.0)) < 1e-6 * L
    assert np.abs(gd - gd.mean(axis=1, keepdims=True)).max() < 1e-8 * gd.max()


def test_time_reversal_at_2_17(oracle_mod):
    T, C, K = 1 << 17, 6, 24
    inp = make_random(1, T, C, K, seed=17, tsd=0.4, dsd=0.4)
    rev = dict(inp)
    rev["emissions"] = np.ascontiguousarray(inp["emissions"][:, ::-1])
    rev["trans"] = np.ascontiguousarray(inp["trans"].T)
    o = oracle_mod.fwd_bwd(inp, nthreads=1)
    r = oracle_mod.fwd_bwd(rev, nthreads=1)
    assert abs(o["logz"][0] - r["logz"][0]) <= 1e-12 * abs(o["logz"][0])
    np.testing.assert_allclose(r["marginals"][0], o["marginals"][0, ::-1], rtol=0, atol=1e-9)
    np.testing.assert_allclose(r["grad_emissions"][0], o["grad_emissions"][0, ::-1], rtol=0,
                               atol=1e-9)
    np.testing.assert_allclose(r["grad_trans"], o["grad_trans"].T, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(r["grad_dur"], o["grad_dur"], rtol=1e-9, atol=1e-9)
    # a segment starting at t in the reversed sequence ends at T - t in the original
    np.testing.assert_allclose(r["boundary"][0, 1:], o["boundary"][0, 1:][::-1], rtol=0,
                               atol=1e-9)
