"""Pin the oracle with identities the mathematics fixes at any size.

* marginals lie in [0, 1] and sum to 1 over labels at every valid position
  (technical summary, section 3: invariants checked at genomic scale);
* log Z from the left equals log Z from the right;
* a duration bias linear in k shifts log Z by lambda * L;
* with centring, adding a per-label constant to the emissions leaves log Z
  unchanged (the baseline absorbs it: technical summary, section 2.C);
* gradient identities: sum_k k * dF/ddur = sum_b w_b L_b;
  sum dF/dtrans = sum dF/ddur - sum_b w_b (one transition fewer than segments);
  with centring, sum_i dF/dx[b,i,c] = 0;
* padding positions (NaN) never reach a result;
* central differences of log Z against every analytic gradient.
"""
import numpy as np
import pytest

from semi_markov_crf_zero_amd.workloads import make_random


@pytest.fixture(scope="module")
def mid_case():
    return make_random(4, 90, 6, 12, seed=3, lengths=[90, 61, 12, 1], sigma=1.5, tsd=0.3, dsd=0.3)


@pytest.mark.parametrize("center", [True, False])
def test_marginal_and_gradient_identities(oracle_mod, mid_case, center):
    w = np.array([1.0, 0.25, -1.5, 3.0])
    out = oracle_mod.fwd_bwd(mid_case, center=center, grad_logz=w)
    L = mid_case["lengths"]
    mu = out["marginals"]
    assert mu.min() > -1e-12 and mu.max() < 1 + 1e-12
    for b in range(4):
        np.testing.assert_allclose(mu[b, :L[b]].sum(axis=1), 1.0, atol=1e-12)
        assert np.all(mu[b, L[b]:] == 0)
        assert np.all(out["grad_emissions"][b, L[b]:] == 0)
        if center:
            np.testing.assert_allclose(out["grad_emissions"][b].sum(axis=0), 0.0, atol=1e-10)
    np.testing.assert_allclose(out["logz"], out["logz_bwd"], rtol=1e-13)
    K = mid_case["dur"].shape[0]
    ks = np.arange(1, K + 1)[:, None]
    assert abs((ks * out["grad_dur"]).sum() - (w * L).sum()) < 1e-10
    assert abs(out["grad_trans"].sum() - (out["grad_dur"].sum() - w.sum())) < 1e-10


def test_duration_shift(oracle_mod, mid_case):
    lam = 0.37
    K = mid_case["dur"].shape[0]
    shifted = dict(mid_case)
    # choose lambda so that dur + lambda*k stays exactly representable in f32
    d = mid_case["dur"].astype(np.float64) + lam * np.arange(1, K + 1)[:, None]
    shifted["dur"] = d.astype(np.float32)
    delta = shifted["dur"].astype(np.float64) - mid_case["dur"].astype(np.float64)
    a = oracle_mod.logz(mid_case)
    b = oracle_mod.logz(shifted)
    # exact per-k shifts actually applied (after f32 rounding) differ from lam*k
    # by < 1e-6; bound the effect by L * max deviation
    dev = np.abs(delta - lam * np.arange(1, K + 1)[:, None]).max()
    np.testing.assert_allclose(b - a, lam * mid_case["lengths"], atol=mid_case["lengths"].max() * dev + 1e-9)


def test_label_shift_invariance_with_centring(oracle_mod, mid_case):
    shifted = dict(mid_case)
    shift = np.array([0.5, -2.0, 1.0, 0.25, 3.0, -0.75], np.float32)
    shifted["emissions"] = (mid_case["emissions"] + shift[None, None, :]).astype(np.float32)
    a = oracle_mod.logz(mid_case, center=True)
    b = oracle_mod.logz(shifted, center=True)
    # f32 rounding of x + shift perturbs the emissions by <= 2^-22 per entry
    np.testing.assert_allclose(a, b, atol=1e-4)
    c = oracle_mod.logz(shifted, center=False)
    assert np.all(np.abs(c - a) > 1e-3)  # without centring the shift is visible


def test_padding_is_ignored(oracle_mod):
    base = make_random(3, 40, 5, 8, seed=9, lengths=[40, 17, 3])
    padded = make_random(3, 40, 5, 8, seed=9, lengths=[40, 17, 3], pad_value=np.nan)
    a = oracle_mod.fwd_bwd(base)
    b = oracle_mod.fwd_bwd(padded)
    for k in ("logz", "grad_emissions", "grad_trans", "grad_dur", "marginals"):
        np.testing.assert_array_equal(a[k], b[k])
    va = oracle_mod.viterbi(base)
    vb = oracle_mod.viterbi(padded)
    for k in va:
        np.testing.assert_array_equal(va[k], vb[k])


def _f32_step(x, h):
    """x + h rounded to float32, and the exact perturbation that was applied."""
    y = np.float32(np.float64(x) + h)
    return y, float(np.float64(y) - np.float64(x))


@pytest.mark.parametrize("center", [True, False])
def test_central_differences_every_element(oracle_mod, center):
    """Tiny case: every gradient element against a central difference of the
    oracle's own log Z (exact applied perturbations; h = 2^-12)."""
    inp = make_random(2, 9, 3, 4, seed=11, lengths=[9, 6], tsd=0.4, dsd=0.4)
    w = np.array([1.0, 0.5])
    out = oracle_mod.fwd_bwd(inp, center=center, grad_logz=w)
    h = 2.0 ** -12

    def F(d):
        return float(np.dot(w, oracle_mod.logz(d, center=center)))

    for key, gkey in (("emissions", "grad_emissions"), ("trans", "grad_trans"), ("dur", "grad_dur")):
        arr = inp[key]
        for idx in np.ndindex(arr.shape):
            if key == "emissions" and idx[1] >= inp["lengths"][idx[0]]:
                continue
            p = dict(inp); m = dict(inp)
            p[key] = arr.copy(); m[key] = arr.copy()
            p[key][idx], dp = _f32_step(arr[idx], h)
            m[key][idx], dm = _f32_step(arr[idx], -h)
            fd = (F(p) - F(m)) / (dp - dm)
            assert abs(fd - out[gkey][idx]) < 5e-7, (key, idx, fd, out[gkey][idx])


def test_directional_derivative_mid(oracle_mod, mid_case):
    """Random directional derivatives on a mid-size case."""
    w = np.ones(4)
    out = oracle_mod.fwd_bwd(mid_case, grad_logz=w)
    rng = np.random.default_rng(1)
    h = 2.0 ** -14
    for key, gkey in (("emissions", "grad_emissions"), ("trans", "grad_trans"), ("dur", "grad_dur")):
        arr = mid_case[key].astype(np.float64)
        v = rng.choice([-1.0, 1.0], size=arr.shape)
        p = dict(mid_case); m = dict(mid_case)
        p[key] = (arr + h * v).astype(np.float32)
        m[key] = (arr - h * v).astype(np.float32)
        dp = p[key].astype(np.float64) - arr
        dm = m[key].astype(np.float64) - arr
        lhs = float(np.sum(oracle_mod.logz(p)) - np.sum(oracle_mod.logz(m)))
        rhs = float(np.sum(out[gkey] * (dp - dm)))
        assert abs(lhs - rhs) < 1e-6 * max(1.0, abs(rhs)), (key, lhs, rhs)
