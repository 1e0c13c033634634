"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on
the same seeded inputs, element by element.

Bars: log Z relative 1e-5; gradients and marginals absolute 1e-4;
Viterbi segmentations identical (smallest-k / smallest-label tie-break).
Shapes cover every workgroup configuration of the library (256/512/1024
threads; C <= 8, <= 32, <= 64, > 64 with 1-4 contraction slices), several
checkpoint intervals and ragged tails, plus the edge cases: K > T, L = 1,
C = 1, K = 1, NaN padding, invalid lengths, non-unit grad weights,
centring off, large emission scales.
"""
import itertools

import numpy as np
import pytest

import oracle
from semi_markov_crf_zero_amd.workloads import make_random
from tests.gpu_util import (assert_fwd_bwd_close, assert_viterbi_equal, gpu_fwd_bwd, gpu_logz,
                            gpu_scan, gpu_viterbi, logz_rel_err, param_excess)

pytestmark = pytest.mark.gpu

# (B, T, C, K, lengths): one per workgroup configuration, ragged tails
SHAPES = [
    (3, 300, 8, 16, [300, 211, 5]),      # 256 threads, C <= 8
    (3, 400, 24, 32, [400, 257, 33]),    # 256 threads, C = 24 (not a power of 2)
    (2, 500, 16, 40, [500, 123]),        # 256 threads, C = 16
    (2, 333, 64, 100, [333, 300]),       # 256 threads, C = 64
    (2, 600, 64, 200, [600, 444]),       # 512 threads
    (2, 300, 100, 70, [300, 151]),       # 512 threads, 2 contraction slices
    (2, 200, 256, 20, [200, 199]),       # 1024 threads, 4 slices
    (2, 150, 200, 50, [150, 77]),        # 1024 threads, C = 200
    (2, 400, 40, 8, [400, 251]),         # 256 threads, odd slice width rounded up (7 -> 8)
    (2, 300, 33, 10, [300, 177]),        # 256 threads, C * (K + P) odd: the e row realigned
    (3, 50, 5, 80, [50, 10, 1]),         # K > T, L = 1
    (2, 64, 1, 8, [64, 63]),             # C = 1
    (2, 90, 6, 1, [90, 40]),             # K = 1 (linear chain)
]


# one per instance of the windowed engine (C <= 32, 256 threads): far
# durations per helper thread A (a multiple of the chunk 2, 4 or 8, at most 48
# in registers) x label bound C in {<=8, <=16, <=32}, the largest A on both
# sides of that bound (C = 16 past it runs on the LDS-ring engine) and the
# two-workgroups-per-compute-unit configuration (C <= 16 with its LDS below
# half the unit's); the C > 32 entries run on the LDS-ring engine.
_WIN64_SKIP = pytest.mark.skip(
    reason="faulted the GPU while C > 32 shapes ran on the windowed engine (cause not "
           "found on the CPU emulation); that engine is now limited to C <= 32 and these "
           "shapes stay off the GPU until the fault is explained")
WINDOW_SHAPES = [
    (2, 300, 8, 40, [300, 177]),         # A = 2,  C <= 8
    (2, 800, 8, 500, [800, 555]),        # A = 24, C <= 8
    (2, 1200, 8, 1000, [1200, 1001]),    # A = 48, C <= 8
    (2, 2600, 8, 1150, [2600, 1777]),    # A = 48, C <= 8, K at the register bound; 2 per unit
    (2, 400, 32, 60, [400, 261]),        # A = 16, C <= 32
    (2, 900, 32, 120, [900, 611]),       # A = 24, C <= 32
    (2, 1100, 16, 500, [1100, 777]),     # A = 48, C <= 16 (genome-like), 2 per unit
    (2, 2000, 16, 576, [2000, 1333]),    # A = 48, C <= 16, K at the register bound
    (2, 2000, 16, 600, [2000, 1500]),    # A would be 56: the LDS-ring engine
    pytest.param((2, 400, 64, 32, [400, 271]), marks=_WIN64_SKIP),
    pytest.param((2, 700, 64, 60, [700, 513]), marks=_WIN64_SKIP),
    pytest.param((2, 600, 48, 160, [600, 389]), marks=_WIN64_SKIP),
]


def _case(B, T, C, K, lengths, seed=0, **kw):
    return make_random(B, T, C, K, seed=seed, lengths=lengths, **kw)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dT%dC%dK%d" % s[:4])
def test_fwd_bwd_shapes(shape):
    B, T, C, K, lengths = shape
    inp = _case(B, T, C, K, lengths, seed=T + C + K, tsd=0.3, dsd=0.3)
    o = oracle.fwd_bwd(inp)
    g = gpu_fwd_bwd(inp)
    errs = assert_fwd_bwd_close(g, o, label=str(shape[:4]))
    print(shape[:4], errs, "logz rel", logz_rel_err(g["logz"], o["logz"]).max())


@pytest.mark.parametrize("shape", WINDOW_SHAPES, ids=lambda s: "B%dT%dC%dK%d" % s[:4])
def test_fwd_bwd_window_instances(shape):
    B, T, C, K, lengths = shape
    inp = _case(B, T, C, K, lengths, seed=3 * T + C + K, tsd=0.3, dsd=0.3)
    o = oracle.fwd_bwd(inp)
    g = gpu_fwd_bwd(inp)
    errs = assert_fwd_bwd_close(g, o, label=str(shape[:4]))
    print(shape[:4], errs)
    assert logz_rel_err(gpu_logz(inp), o["logz"]).max() <= 1e-5


@pytest.mark.parametrize("C,K", list(itertools.product([1, 2, 3], [1, 2, 3, 4])))
def test_fwd_bwd_enumeration_grid(C, K):
    """The oracle is pinned to explicit enumeration on exactly this grid."""
    T = 7 if C == 3 else 8
    for center in (True, False):
        inp = _case(3, T, C, K, [T, 4, 1], seed=C * 10 + K, tsd=0.5, dsd=0.5)
        o = oracle.fwd_bwd(inp, center=center, grad_logz=np.array([1.0, -0.5, 2.0]))
        g = gpu_fwd_bwd(inp, center=center, w=[1.0, -0.5, 2.0])
        assert_fwd_bwd_close(g, o, tol_logz=1e-6, tol=1e-5, label=(C, K, center))


@pytest.mark.parametrize("ckpt", [1, 3, 16, 0, 97, 400])
def test_checkpoint_interval_invariance(ckpt):
    inp = _case(3, 400, 12, 16, [400, 399, 130], seed=5, tsd=0.3, dsd=0.3)
    o = oracle.fwd_bwd(inp)
    g = gpu_fwd_bwd(inp, ckpt=ckpt)
    assert_fwd_bwd_close(g, o, label=ckpt)
    ref = gpu_fwd_bwd(inp, ckpt=0)
    for k in ("grad_emissions", "marginals"):
        assert np.abs(g[k] - ref[k]).max() < 1e-5
    for k in ("grad_trans", "grad_dur"):
        assert param_excess(g[k], ref[k], 1e-5) <= 1.0, k
    assert np.abs(g["logz"] - ref["logz"]).max() <= 1e-6 * np.abs(ref["logz"]).max()


def test_weights_and_no_center():
    inp = _case(3, 257, 10, 24, [257, 256, 100], seed=7)
    w = np.array([0.5, -1.25, 3.0])
    for center in (True, False):
        o = oracle.fwd_bwd(inp, center=center, grad_logz=w)
        g = gpu_fwd_bwd(inp, center=center, w=w)
        assert_fwd_bwd_close(g, o, label=center)


def test_nan_padding_is_never_read():
    clean = _case(3, 200, 8, 16, [200, 77, 9], seed=9)
    padded = _case(3, 200, 8, 16, [200, 77, 9], seed=9, pad_value=np.nan)
    a = gpu_fwd_bwd(clean)
    b = gpu_fwd_bwd(padded)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    va, vb = gpu_viterbi(clean), gpu_viterbi(padded)
    for k in va:
        assert np.array_equal(va[k], vb[k]), k


def test_invalid_lengths():
    """lengths outside [1, T]: NaN log Z, zero gradient rows, excluded from
    the parameter gradients (compared with the valid sequence alone)."""
    base = _case(3, 60, 4, 8, [60, 60, 23], seed=11)
    bad = dict(base)
    bad["lengths"] = np.array([0, 61, 23], np.int32)
    g = gpu_fwd_bwd(bad)
    assert np.isnan(g["logz"][0]) and np.isnan(g["logz"][1])
    assert np.all(g["grad_emissions"][:2] == 0) and np.all(g["marginals"][:2] == 0)
    only = dict(base)
    for k in ("emissions",):
        only[k] = base[k][2:3]
    only["lengths"] = np.array([23], np.int32)
    o = oracle.fwd_bwd(only)
    assert abs(g["logz"][2] - o["logz"][0]) <= 1e-5 * abs(o["logz"][0])
    assert np.abs(g["grad_trans"] - o["grad_trans"]).max() <= 1e-4
    assert np.abs(g["grad_dur"] - o["grad_dur"]).max() <= 1e-4
    assert np.abs(g["grad_emissions"][2] - o["grad_emissions"][0]).max() <= 1e-4
    lz = gpu_logz(bad)
    assert np.isnan(lz[0]) and np.isnan(lz[1])
    v = gpu_viterbi(bad)
    assert np.isnan(v["best_score"][0]) and v["num_segs"][0] == 0 and np.all(v["seg_start"][0] == -1)


@pytest.mark.parametrize("sigma", [10.0, 100.0])
def test_large_emission_scales(sigma):
    inp = _case(2, 300, 8, 24, [300, 181], seed=13, sigma=sigma, tsd=1.0, dsd=1.0)
    o = oracle.fwd_bwd(inp)
    g = gpu_fwd_bwd(inp)
    assert_fwd_bwd_close(g, o, label=sigma)
    assert_viterbi_equal(gpu_viterbi(inp), oracle.viterbi(inp), label=sigma)


@pytest.mark.parametrize("sigma", [1.0, 100.0])
def test_duration_posteriors_many_lags(sigma):
    """K = 200 with 16 labels a group: the duration kernel's lag blocks of 16.
    At emission scale 100 the scores swing by hundreds of nats within a
    64-start tile, so labels take the direct path (an exponential per
    cell); at scale 1 the factorised path."""
    inp = _case(2, 700, 20, 200, [700, 433], seed=29, sigma=sigma, tsd=1.0, dsd=1.0)
    o = oracle.fwd_bwd(inp)
    assert_fwd_bwd_close(gpu_fwd_bwd(inp), o, label=sigma)


@pytest.mark.parametrize("sigma", [10.0, 100.0])
def test_large_emission_scales_lds_ring(sigma):
    """C = 48 runs the LDS-ring engine: frequent rebases, applied a step
    late (and at once on the steps that store a checkpoint record)."""
    inp = _case(2, 400, 48, 30, [400, 263], seed=17, sigma=sigma, tsd=1.0, dsd=1.0)
    o = oracle.fwd_bwd(inp)
    assert_fwd_bwd_close(gpu_fwd_bwd(inp), o, label=sigma)
    assert_fwd_bwd_close(gpu_fwd_bwd(inp, ckpt=64), o, label=(sigma, 64))


@pytest.mark.parametrize("C", [24, 40])
def test_large_emissions_with_burn_in(C):
    """Intervals of at least 8K positions start with a burn-in whose last
    step stores the chunk's start record; with emission scale 30 labels
    rebase often, also on that step (windowed engine at C = 24, LDS-ring at
    C = 40)."""
    inp = _case(2, 800, C, 12, [800, 555], seed=23, sigma=30.0, tsd=1.0, dsd=1.0)
    o = oracle.fwd_bwd(inp)
    assert_fwd_bwd_close(gpu_fwd_bwd(inp, ckpt=128), o, label=(C, 128))


def test_deterministic_bitwise():
    inp = _case(3, 500, 16, 40, [500, 300, 77], seed=17)
    a = gpu_fwd_bwd(inp)
    b = gpu_fwd_bwd(inp)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("shape", SHAPES[:8], ids=lambda s: "B%dT%dC%dK%d" % s[:4])
def test_logz_fwd(shape):
    B, T, C, K, lengths = shape
    inp = _case(B, T, C, K, lengths, seed=1 + T)
    o = oracle.logz(inp)
    g = gpu_logz(inp)
    assert logz_rel_err(g, o).max() <= 1e-5


@pytest.mark.parametrize("C,T", [(1, 50), (3, 1000), (16, 4097), (24, 777), (64, 3000), (256, 300)])
def test_cumulative_scores(C, T):
    inp = _case(3, T, C, 4, [T, T // 2 + 1, 1], seed=C, sigma=2.0)
    for center in (True, False):
        nu_o, S_o = oracle.prefix(inp, center=center)
        nu_g, S_g = gpu_scan(inp, center=center)
        np.testing.assert_allclose(nu_g, nu_o, rtol=1e-12, atol=1e-12)
        # S rows beyond L repeat row L on both sides
        np.testing.assert_allclose(S_g, S_o, rtol=1e-11, atol=1e-9)
        if center:
            L = inp["lengths"]
            for b in range(3):
                assert np.abs(S_g[b, L[b]]).max() < 1e-9 * max(1, L[b])


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dT%dC%dK%d" % s[:4])
def test_viterbi_shapes(shape):
    B, T, C, K, lengths = shape
    inp = _case(B, T, C, K, lengths, seed=2 * T + C, tsd=0.3, dsd=0.3)
    assert_viterbi_equal(gpu_viterbi(inp), oracle.viterbi(inp), label=shape[:4])


# Shapes whose label groups stop narrowing at 512 threads (a lane would
# otherwise hold more than 16 durations): the 512-thread decoder instances.
VIT_512_SHAPES = [
    (2, 700, 16, 300, [700, 433]),       # 32-lane groups, 10 durations per lane
    (2, 900, 8, 600, [900, 610]),        # 64-lane groups, 10 durations per lane
    (2, 500, 20, 200, [500, 321]),       # 16-lane groups, 13 durations, 2 labels per lane
]


@pytest.mark.parametrize("shape", VIT_512_SHAPES, ids=lambda s: "B%dT%dC%dK%d" % s[:4])
def test_viterbi_512_thread_groups(shape):
    B, T, C, K, lengths = shape
    inp = _case(B, T, C, K, lengths, seed=3 * T + C, tsd=0.3, dsd=0.3)
    assert_viterbi_equal(gpu_viterbi(inp), oracle.viterbi(inp), label=shape[:4])


def test_viterbi_serial_decoder_shape():
    """C = 8, K = 1100: more durations per lane than the parallel-in-time
    decoder holds, so the one-workgroup-per-sequence decoder runs."""
    inp = _case(2, 1500, 8, 1100, [1500, 1200], seed=77, tsd=0.3, dsd=0.3)
    assert_viterbi_equal(gpu_viterbi(inp), oracle.viterbi(inp), label="serial decoder")


def test_viterbi_chunks_that_never_forget():
    """Switching labels costs 50, so the best path never switches and each
    label's score depends on every earlier position: no chunk's burn-in
    reaches a start-independent state, every boundary check fails, and only
    the in-order repair makes the decoding exact."""
    rng = np.random.default_rng(5)
    B, T, C, K = 2, 5000, 3, 5
    x = (0.01 * rng.standard_normal((B, T, C))).astype(np.float32)
    tr = np.full((C, C), -50.0, np.float32)
    np.fill_diagonal(tr, 0.0)
    du = (0.01 * rng.standard_normal((K, C))).astype(np.float32)
    inp = dict(emissions=x, lengths=np.array([T, 3777], np.int32), trans=tr, dur=du)
    g, o = gpu_viterbi(inp), oracle.viterbi(inp)
    assert_viterbi_equal(g, o, label="sticky")
    assert np.all(g["seg_label"][0, :g["num_segs"][0]] == g["seg_label"][0, 0])


def test_viterbi_tie_break_zero_potentials():
    """Every segmentation ties: the rule yields L unit segments of label 0."""
    for (C, K, T) in [(3, 5, 40), (16, 32, 100), (64, 8, 33)]:
        inp = dict(emissions=np.zeros((2, T, C), np.float32),
                   lengths=np.array([T, T - 7], np.int32),
                   trans=np.zeros((C, C), np.float32), dur=np.zeros((K, C), np.float32))
        g = gpu_viterbi(inp)
        for b, L in enumerate([T, T - 7]):
            assert g["num_segs"][b] == L
            assert np.all(g["seg_len"][b, :L] == 1) and np.all(g["seg_label"][b, :L] == 0)
            assert np.all(g["seg_start"][b, :L] == np.arange(L)) and np.all(g["seg_start"][b, L:] == -1)
        assert_viterbi_equal(g, oracle.viterbi(inp))


@pytest.mark.parametrize("C,K", list(itertools.product([1, 2, 3], [1, 2, 3, 4])))
def test_viterbi_enumeration_grid(C, K):
    T = 7 if C == 3 else 8
    for center in (True, False):
        inp = _case(3, T, C, K, [T, 4, 1], seed=100 + C * 10 + K, tsd=0.5, dsd=0.5)
        assert_viterbi_equal(gpu_viterbi(inp, center), oracle.viterbi(inp, center), label=(C, K))


@pytest.mark.parametrize("C,T,ckpt", [(4, 2048, 64), (4, 2048, 0), (48, 1024, 64),
                                      (96, 1024, 64)])
def test_fwd_bwd_sticky_transitions_redo(C, T, ckpt):
    """Off-diagonal transitions of -50: the chain stays in one label for long
    runs, so the direction of each interval's state depends on the far past
    and a neutral start does not match its predecessor's end: the
    parallel-in-time sweeps go through their verification failures, redo
    sweeps, the in-order repair of the chunks still inconsistent after the
    parallel passes and the in-order correction of the interval
    normalisers.  C = 4, 48 and 96 take the windowed, 64-label and
    256-label sweep engines (the last with its float64 variant at the full
    bar).  Every element against the oracle.

    The float32-ring engine (C = 96 by default) meets the bar on log Z,
    marginals and emission gradients here, but not the one-ulp bar of the
    parameter gradients: on a chain that stays in one label the rounding
    of the state's scale adds up along the run (a random walk of one float32
    rounding per position), and grad_trans / grad_dur sum the posteriors of
    the whole run (values near 1000 here).  Its bar for those two is
    sqrt(T) float32 roundings of the value; measured: 0.4 of it."""
    inp = _case(2, T, C, 16, [T, T - 547], seed=11, tsd=0.0, dsd=0.3)
    trans = np.full((C, C), -50.0, np.float32)
    np.fill_diagonal(trans, 0.0)
    inp["trans"] = trans
    o = oracle.fwd_bwd(inp)
    g = gpu_fwd_bwd(inp, ckpt=ckpt, float64=C > 64)
    errs = assert_fwd_bwd_close(g, o, label=("sticky", C, ckpt))
    print("sticky", C, ckpt, errs)
    if C > 64:
        f = gpu_fwd_bwd(inp, ckpt=ckpt)
        errs = assert_fwd_bwd_close(f, o, label=("sticky float32 ring", C, ckpt),
                                    param_rel=np.sqrt(T) * 2.0 ** -24)
        print("sticky float32 ring", C, ckpt, errs)
    assert_viterbi_equal(gpu_viterbi(inp), oracle.viterbi(inp), label="sticky")
