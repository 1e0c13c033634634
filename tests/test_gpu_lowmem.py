"""GPU parity of the low-memory forward-backward (SEMICRF_LOW_MEMORY): the
sweeps keep only the checkpoint records and the posterior pass replays the
intervals window by window from those records -- the recomputation between
checkpoints of "Streaming Structured Inference with Flash-SemiCRF" (abstract:
working memory sublinear in sequence length; technical summary, section
2.C).  Every element against the float64 oracle, on shapes that span several
windows on both sweep engines (windowed C <= 32, LDS-ring C > 32 at 256, 512
and 1024 threads), ragged lengths, an interval below K (raised to K), K > T,
invalid lengths, weights, centring off, and the named workloads; extreme
against its golden file here, and element by element against the oracle in
test_gpu_workloads.py."""
import os

import numpy as np
import pytest

import oracle
from semi_markov_crf_zero_amd import binding as bd
from semi_markov_crf_zero_amd.workloads import make_inputs, make_random
from tests.gpu_util import TOL_GRAD, assert_fwd_bwd_close, gpu_fwd_bwd, logz_rel_err, param_excess

pytestmark = pytest.mark.gpu

# (B, T, C, K, lengths, interval): windows of ceil(sqrt(#intervals)) intervals
SHAPES = [
    (2, 3000, 8, 16, [3000, 1777], 0),       # windowed engine, 14 intervals, 4 windows
    (3, 2500, 24, 32, [2500, 2499, 301], 0),  # windowed, C = 24, a short sequence
    (2, 2000, 64, 40, [2000, 1234], 0),       # LDS-ring 256 threads, 8 intervals, 3 windows
    (1, 5000, 100, 10, [4999], 0),            # 512 threads, 2 contraction slices
    (2, 800, 256, 20, [800, 513], 0),         # 1024 threads (weights streamed)
    (2, 1500, 12, 48, [1500, 1100], 20),      # interval 20 < K: raised to K = 48
    (2, 900, 16, 60, [900, 899], 100),        # given interval, 9 intervals
    (3, 50, 5, 80, [50, 10, 1], 0),           # K > T: one interval
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dT%dC%dK%d" % s[:4])
def test_low_memory_shapes(shape):
    B, T, C, K, lengths, ckpt = shape
    inp = make_random(B, T, C, K, seed=T + C + K, lengths=lengths, tsd=0.3, dsd=0.3)
    o = oracle.fwd_bwd(inp)
    g = gpu_fwd_bwd(inp, ckpt=ckpt, low_memory=True)
    errs = assert_fwd_bwd_close(g, o, label=("lowmem",) + shape[:4])
    f = gpu_fwd_bwd(inp, ckpt=ckpt)  # the default path on the same input
    for k in ("grad_emissions", "marginals", "boundary"):
        assert np.abs(g[k] - f[k]).max() <= 1e-5, k
    print(shape[:4], errs)


def test_low_memory_invalid_lengths_weights_no_center():
    inp = make_random(4, 700, 10, 24, seed=9, lengths=[700, 0, 699, 800], pad_value=np.nan)
    inp["lengths"] = np.array([700, 0, 699, 800], np.int32)  # 0 and 800 > T are invalid
    w = np.array([0.5, 2.0, -1.25, 3.0])
    for center in (True, False):
        o = oracle.fwd_bwd(inp, center=center, grad_logz=w)
        g = gpu_fwd_bwd(inp, center=center, w=w, ckpt=64, low_memory=True)
        assert_fwd_bwd_close(g, o, label=("lowmem-invalid", center))
        assert np.isnan(g["logz"][1]) and np.isnan(g["logz"][3])
        assert np.all(g["grad_emissions"][[1, 3]] == 0)


@pytest.mark.parametrize("name", ["tiny", "nlp", "speech", "genome"])
def test_low_memory_workloads(name):
    inp = make_inputs(name)
    g = gpu_fwd_bwd(inp, low_memory=True)
    o = oracle.fwd_bwd(inp)
    errs = assert_fwd_bwd_close(g, o, label=("lowmem", name))
    print(name, errs)


def test_low_memory_extreme_golden():
    from tests.golden.make_golden import input_digest
    inp = make_inputs("extreme")
    gold = np.load(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                "extreme.npz"), allow_pickle=False)
    assert input_digest(inp) == str(gold["input_sha256"])
    g = gpu_fwd_bwd(inp, low_memory=True)
    assert logz_rel_err(g["logz"], gold["logz"]).max() <= 1e-5
    assert param_excess(g["grad_trans"], gold["grad_trans"]) <= 1.0
    assert param_excess(g["grad_dur"], gold["grad_dur"]) <= 1.0
    rows = gold["rows"]
    bidx = np.arange(inp["B"])[:, None]
    for k, gk in (("marginals", "marginals_rows"), ("grad_emissions", "grad_rows"),
                  ("boundary", "boundary_rows")):
        e = float(np.abs(g[k][bidx, rows] - gold[gk]).max())
        assert e <= TOL_GRAD, (k, e)
    blk = int(gold["block"])
    for k, gk in (("marginals", "marginals_blocks"), ("grad_emissions", "grad_blocks")):
        L = int(inp["lengths"][0])
        nb = gold[gk].shape[1]
        sums = np.stack([g[k][0, i * blk:min((i + 1) * blk, L)].sum(axis=0) for i in range(nb)])
        assert np.abs(sums - gold[gk][0]).max() <= TOL_GRAD * blk, k
    ws_low = bd.semicrf_workspace_size(bd.OP_FWD_BWD, 1, inp["T"], inp["C"], inp["K"],
                                       bd.LOW_MEMORY)
    ws_all = bd.semicrf_workspace_size(bd.OP_FWD_BWD, 1, inp["T"], inp["C"], inp["K"], 0)
    print("extreme workspace: low-memory %.0f MB, default %.0f MB" % (ws_low / 1e6, ws_all / 1e6))
    assert ws_low < ws_all / 3
