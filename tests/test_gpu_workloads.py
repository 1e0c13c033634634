"""GPU parity on the five named workloads, in the launch configuration that
bench.py times (default checkpoint interval, library-chosen workgroups).

tiny and NLP: element-by-element against the oracle run in the test.
speech, genome, extreme: against tests/golden/<name>.npz, written by
tests/golden/make_golden.py from the oracle alone (log Z, parameter
gradients, sampled rows of marginals / emission gradients / cumulative
scores, the complete Viterbi segmentation), plus properties checked over
every position: marginals in [0, 1] summing to 1 over labels, and (with
centring) emission gradients summing to 0 over time for every label.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from semi_markov_crf_zero_amd import binding as bd
from semi_markov_crf_zero_amd.workloads import make_inputs
from tests.golden.make_golden import input_digest
from tests.gpu_util import (TOL_GRAD, assert_fwd_bwd_close, assert_viterbi_equal, gpu_fwd_bwd,
                            gpu_scan, gpu_viterbi, logz_rel_err, param_excess, to_dev)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.mark.parametrize("name", ["tiny", "nlp"])
def test_small_workloads_full(name):
    inp = make_inputs(name)
    o = oracle.fwd_bwd(inp)
    g = gpu_fwd_bwd(inp)
    errs = assert_fwd_bwd_close(g, o, label=name)
    print(name, errs)
    assert_viterbi_equal(gpu_viterbi(inp), oracle.viterbi(inp), label=name)


def _properties(inp, out):
    mu = out["marginals"]
    L = inp["lengths"]
    assert mu.min() >= -TOL_GRAD and mu.max() <= 1 + TOL_GRAD
    for b in range(inp["B"]):
        s = mu[b, :L[b]].sum(axis=1)
        assert np.abs(s - 1).max() <= TOL_GRAD, (b, np.abs(s - 1).max())
        assert np.all(mu[b, L[b]:] == 0)
        col = out["grad_emissions"][b, :L[b]].sum(axis=0)
        assert np.abs(col).max() <= 2e-3 * max(1.0, L[b] / 1000.0)


@pytest.mark.parametrize("name", ["speech", "genome", "extreme"])
def test_large_workloads_golden(name):
    path = os.path.join(GOLDEN, name + ".npz")
    gold = np.load(path, allow_pickle=False)
    inp = make_inputs(name)
    assert input_digest(inp) == str(gold["input_sha256"]), "input generator drifted"
    t = to_dev(inp)
    out = bd.semicrf_fwd_bwd(t["emissions"], t["lengths"], t["trans"], t["dur"],
                             want_marginals=True)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy().astype(np.float64) for k, v in out.items()}
    rel = logz_rel_err(g["logz"], gold["logz"])
    assert rel.max() <= 1e-5, rel
    e_tr = np.abs(g["grad_trans"] - gold["grad_trans"]).max()
    e_du = np.abs(g["grad_dur"] - gold["grad_dur"]).max()
    x_tr = param_excess(g["grad_trans"], gold["grad_trans"])
    x_du = param_excess(g["grad_dur"], gold["grad_dur"])
    rows = gold["rows"]
    bidx = np.arange(inp["B"])[:, None]
    e_mu = np.abs(g["marginals"][bidx, rows] - gold["marginals_rows"]).max()
    e_gx = np.abs(g["grad_emissions"][bidx, rows] - gold["grad_rows"]).max()
    print(name, "logz rel %.2e trans %.2e dur %.2e mu %.2e gx %.2e" % (rel.max(), e_tr, e_du, e_mu, e_gx))
    assert x_tr <= 1.0 and x_du <= 1.0, (e_tr, x_tr, e_du, x_du)
    assert e_mu <= TOL_GRAD and e_gx <= TOL_GRAD
    np.testing.assert_allclose(g["marginals"].sum(axis=1), gold["colsum_marginals"],
                               atol=TOL_GRAD * inp["T"] / 100)
    _properties(inp, g)
    del g, out
    # cumulative scores at sampled rows
    nu, S = gpu_scan(inp)
    np.testing.assert_allclose(nu, gold["nu"], rtol=1e-12, atol=1e-12)
    # float64 running sums of T terms: each addition rounds by at most u*|partial sum|,
    # so the two summation orders agree within 2u*T*max|S| (u = 2^-53)
    s_tol = 2.0 ** -52 * inp["T"] * max(1.0, float(np.abs(gold["S_rows"]).max()))
    np.testing.assert_allclose(S[bidx, rows[:, ::4]], gold["S_rows"], rtol=0, atol=s_tol)
    np.testing.assert_allclose(S[np.arange(inp["B"]), inp["lengths"]], gold["S_last"], atol=s_tol)
    del S
    # Viterbi: the complete segmentation
    v = gpu_viterbi(inp)
    n = gold["vit_num"]
    assert np.array_equal(v["num_segs"], n), (v["num_segs"], n, gold["vit_margin"])
    for b in range(inp["B"]):
        for k, gk in (("seg_start", "vit_start"), ("seg_len", "vit_len"), ("seg_label", "vit_label")):
            assert np.array_equal(v[k][b, :n[b]], gold[gk][b, :n[b]]), (b, k, gold["vit_margin"][b])
        assert np.all(v["seg_start"][b, n[b]:] == -1)
    np.testing.assert_allclose(v["best_score"], gold["vit_score"], rtol=1e-6)
