"""GPU parity of the low-memory Viterbi decoder (SEMICRF_LOW_MEMORY): the
parallel sweeps keep only each chunk's start state, and the decisions are
recomputed window by window from the end, each window followed back by one
walk per sequence (technical summary, section 2.C: recomputation between
checkpoints; abstract: working memory sublinear in sequence length).  The
segmentation must be the oracle's (tie rule R13) and the same as the
whole-sequence decoder's, on shapes with many windows, ragged and invalid
lengths, K large next to the chunk, sticky transitions (every chunk
repaired), the genome workload and the extreme workload's golden
segmentation (T = 2^20)."""
import os

import numpy as np
import pytest

import oracle
from semi_markov_crf_zero_amd.workloads import make_inputs, make_random
from tests.gpu_util import assert_viterbi_equal, gpu_viterbi

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# (B, T, C, K, lengths)
SHAPES = [
    (2, 3000, 8, 16, [3000, 1777]),         # 47 chunks, 7 windows
    (3, 2500, 24, 32, [2500, 2499, 301]),   # a short sequence ends in an early window
    (2, 2000, 64, 40, [2000, 1234]),
    (1, 5000, 100, 10, [4999]),             # 256 chunks of 64 positions: 16 windows
    (2, 800, 256, 20, [800, 513]),
    (2, 4000, 16, 120, [4000, 3999]),       # K = 120: chunks of 2K, the chunk before a window
    (3, 50, 5, 80, [50, 10, 1]),            # K > T: one chunk, the flag changes nothing
]


def _same(a, b, label):
    for k in ("num_segs", "seg_start", "seg_len", "seg_label"):
        assert np.array_equal(a[k], b[k]), (label, k)
    assert np.array_equal(np.isnan(a["best_score"]), np.isnan(b["best_score"])), label
    ok = ~np.isnan(b["best_score"])
    assert np.array_equal(a["best_score"][ok], b["best_score"][ok]), label


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dT%dC%dK%d" % s[:4])
def test_viterbi_low_memory_shapes(shape):
    B, T, C, K, lengths = shape
    print("case", shape[:4], flush=True)
    inp = make_random(B, T, C, K, seed=3 * T + C + K, lengths=lengths, tsd=0.3, dsd=0.3)
    g = gpu_viterbi(inp, low_memory=True)
    assert_viterbi_equal(g, oracle.viterbi(inp), label=("lowmem",) + shape[:4])
    _same(g, gpu_viterbi(inp), shape[:4])


def test_viterbi_low_memory_invalid_lengths_and_sticky_chunks():
    print("case invalid", flush=True)
    inp = make_random(4, 700, 10, 24, seed=19, lengths=[700, 0, 699, 800])
    inp["lengths"] = np.array([700, 0, 699, 800], np.int32)  # 0 and 800 > T are invalid
    g = gpu_viterbi(inp, low_memory=True)
    assert_viterbi_equal(g, oracle.viterbi(inp), label="lowmem-invalid")
    assert np.isnan(g["best_score"][1]) and np.isnan(g["best_score"][3])
    assert g["num_segs"][1] == 0 and g["num_segs"][3] == 0
    # a label that never forgets: every chunk start differs from its
    # predecessor's end by more than a constant, so every chunk is repaired
    print("case sticky", flush=True)
    inp = make_random(2, 2400, 6, 12, seed=23, lengths=[2400, 2000], tsd=0.1, dsd=0.1)
    tr = np.full((6, 6), -50.0, np.float32)
    np.fill_diagonal(tr, 0.0)
    inp["trans"] = tr
    g = gpu_viterbi(inp, low_memory=True)
    assert_viterbi_equal(g, oracle.viterbi(inp), label="lowmem-sticky")
    _same(g, gpu_viterbi(inp), "sticky")


def test_viterbi_low_memory_genome_matches_whole_decoder():
    print("case genome", flush=True)
    inp = make_inputs("genome")
    _same(gpu_viterbi(inp, low_memory=True), gpu_viterbi(inp), "genome")


def test_viterbi_low_memory_extreme_golden():
    print("case extreme", flush=True)
    inp = make_inputs("extreme")
    gold = np.load(os.path.join(GOLDEN, "extreme.npz"), allow_pickle=False)
    v = gpu_viterbi(inp, low_memory=True)
    n = gold["vit_num"]
    assert np.array_equal(v["num_segs"], n), (v["num_segs"], n)
    for b in range(inp["B"]):
        for k, gk in (("seg_start", "vit_start"), ("seg_len", "vit_len"), ("seg_label", "vit_label")):
            assert np.array_equal(v[k][b, :n[b]], gold[gk][b, :n[b]]), (b, k)
        assert np.all(v["seg_start"][b, n[b]:] == -1)
    np.testing.assert_allclose(v["best_score"], gold["vit_score"], rtol=1e-6)
